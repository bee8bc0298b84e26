"""Seeded synthetic inputs for the five decode workloads.

This module only draws numbers: it holds none of the model's arithmetic, and
both the HIP library's tests/benchmark and the CPU oracle take their inputs
from here.  Weights are random (the trained checkpoint is not available), in
the Hugging Face GPT-2 layout (Conv1D matrices as [input][output]); every step
streams every weight whatever the token, so random weights move exactly the
bytes of real ones.

Recipe (one numpy PCG64 stream per seed, float64 normals cast to float32,
tensors drawn in the fixed order wte, wpe, then per layer in Hugging Face order
ln_1.weight, ln_1.bias, attn.c_attn.weight, attn.c_attn.bias, attn.c_proj.weight,
attn.c_proj.bias, ln_2.weight, ln_2.bias, mlp.c_fc.weight, mlp.c_fc.bias,
mlp.c_proj.weight, mlp.c_proj.bias, then ln_f.weight, ln_f.bias):

- tiny  : matrices N(0, 0.02); LayerNorm gamma = 1, beta = 0; biases 0 (not drawn)
- small : matrices N(0, 0.02); gamma = 1 + N(0, 0.05); beta and biases N(0, 0.01)

Prompt ids: PCG64(prompt_seed).integers(0, vocab, n_prompt).
"""
from dataclasses import dataclass, replace
import functools

import numpy as np


@dataclass(frozen=True)
class Config:
    key: int
    name: str
    n_layer: int
    n_embd: int
    n_head: int
    n_positions: int
    vocab: int
    init: str            # "tiny" or "small"
    wdtype: str          # "fp32", "fp16" or "int4"
    n_prompt: int
    n_new: int
    weight_seed: int
    prompt_seed: int
    ln_eps: float = 1e-5
    q4_group: int = 32

    @property
    def head_dim(self) -> int:
        return self.n_embd // self.n_head

    @property
    def n_steps(self) -> int:
        """Forward passes of one run: the prompt at positions 0..n_prompt-1, then
        one pass per generated id that is fed back (the last id is not fed)."""
        return self.n_prompt + self.n_new - 1


TINY = dict(n_layer=2, n_embd=128, n_head=4, n_positions=64, vocab=512, init="tiny")
SMALL = dict(n_layer=12, n_embd=768, n_head=12, n_positions=1024, vocab=50257, init="small")

CONFIGS = {
    1: Config(1, "tiny-fp32", **TINY, wdtype="fp32", n_prompt=8, n_new=16,
              weight_seed=1001, prompt_seed=2001),
    2: Config(2, "gpt2-124m-fp32", **SMALL, wdtype="fp32", n_prompt=10, n_new=60,
              weight_seed=1002, prompt_seed=2002),
    3: Config(3, "gpt2-124m-fp16w", **SMALL, wdtype="fp16", n_prompt=10, n_new=60,
              weight_seed=1002, prompt_seed=2003),
    4: Config(4, "gpt2-124m-int4w", **SMALL, wdtype="int4", n_prompt=10, n_new=60,
              weight_seed=1002, prompt_seed=2004),
    5: Config(5, "gpt2-124m-fp32-long", **SMALL, wdtype="fp32", n_prompt=8, n_new=1017,
              weight_seed=1002, prompt_seed=2005),
}

BLOCK_NAMES = ("ln_1.weight", "ln_1.bias", "attn.c_attn.weight", "attn.c_attn.bias",
               "attn.c_proj.weight", "attn.c_proj.bias", "ln_2.weight", "ln_2.bias",
               "mlp.c_fc.weight", "mlp.c_fc.bias", "mlp.c_proj.weight", "mlp.c_proj.bias")


def tensor_shapes(cfg: Config):
    """(name, shape) in draw order."""
    E, F, V, P = cfg.n_embd, 4 * cfg.n_embd, cfg.vocab, cfg.n_positions
    block = {"ln_1.weight": (E,), "ln_1.bias": (E,), "attn.c_attn.weight": (E, 3 * E),
             "attn.c_attn.bias": (3 * E,), "attn.c_proj.weight": (E, E),
             "attn.c_proj.bias": (E,), "ln_2.weight": (E,), "ln_2.bias": (E,),
             "mlp.c_fc.weight": (E, F), "mlp.c_fc.bias": (F,), "mlp.c_proj.weight": (F, E),
             "mlp.c_proj.bias": (E,)}
    out = [("wte.weight", (V, E)), ("wpe.weight", (P, E))]
    for l in range(cfg.n_layer):
        out += [(f"h.{l}.{n}", block[n]) for n in BLOCK_NAMES]
    out += [("ln_f.weight", (E,)), ("ln_f.bias", (E,))]
    return out


class Model:
    """Host fp32 parameters (dict name -> array) plus the config they belong to."""

    def __init__(self, cfg: Config, tensors: dict):
        self.cfg = cfg
        self.t = tensors

    def flat_tensors(self):
        return [self.t[n] for n, _ in tensor_shapes(self.cfg)]

    def with_cfg(self, cfg: Config) -> "Model":
        return Model(cfg, self.t)


def _draw(cfg: Config) -> dict:
    rng = np.random.Generator(np.random.PCG64(cfg.weight_seed))
    out = {}
    for name, shape in tensor_shapes(cfg):
        leaf = name.split(".")[-2] + "." + name.split(".")[-1] if name.startswith("h.") else name
        is_ln = leaf.startswith("ln_") or name.startswith("ln_f")
        is_bias = name.endswith(".bias")
        if is_ln and name.endswith(".weight"):
            if cfg.init == "tiny":
                a = np.ones(shape, np.float32)
            else:
                a = (1.0 + rng.normal(0.0, 0.05, shape)).astype(np.float32)
        elif is_bias:
            if cfg.init == "tiny":
                a = np.zeros(shape, np.float32)
            else:
                a = rng.normal(0.0, 0.01, shape).astype(np.float32)
        else:
            a = rng.normal(0.0, 0.02, shape).astype(np.float32)
        out[name] = a
    return out


@functools.lru_cache(maxsize=2)
def _weights(weight_seed: int, init: str, shape_key: tuple) -> dict:
    n_layer, n_embd, n_head, n_positions, vocab = shape_key
    cfg = Config(0, "draw", n_layer, n_embd, n_head, n_positions, vocab, init, "fp32", 1, 1,
                 weight_seed, 0)
    return _draw(cfg)


def make_model(cfg) -> Model:
    if isinstance(cfg, int):
        cfg = CONFIGS[cfg]
    key = (cfg.n_layer, cfg.n_embd, cfg.n_head, cfg.n_positions, cfg.vocab)
    return Model(cfg, _weights(cfg.weight_seed, cfg.init, key))


def make_prompt(cfg) -> np.ndarray:
    if isinstance(cfg, int):
        cfg = CONFIGS[cfg]
    rng = np.random.Generator(np.random.PCG64(cfg.prompt_seed))
    return rng.integers(0, cfg.vocab, cfg.n_prompt).astype(np.int32)


def variant(cfg: Config, **kw) -> Config:
    return replace(cfg, **kw)


# ---------------------------------------------------------------- tokenizer
def synthetic_text(seed: int, n_words: int = 20000) -> str:
    """Seeded English-like text for training and exercising a byte-level BPE:
    pseudo-words from a Zipf-weighted lexicon, some capitalised or with an
    ending such as 's, 't, 're, 've, 'm, 'll or 'd, numbers, punctuation, and
    spaces, runs of spaces, tabs and newlines between them."""
    rng = np.random.Generator(np.random.PCG64(seed))
    letters = np.array(list("etaoinshrdlcumwfgypbvkjxqz"))
    freq = np.array([12.7, 9.1, 8.2, 7.5, 7.0, 6.7, 6.3, 6.1, 6.0, 4.3, 4.0, 2.8, 2.8, 2.4, 2.4, 2.2, 2.0,
                     2.0, 1.9, 1.5, 1.0, 0.8, 0.15, 0.15, 0.1, 0.07])
    freq = freq / freq.sum()
    lexicon = ["".join(rng.choice(letters, size=int(rng.integers(1, 9)), p=freq)) for _ in range(3000)]
    zipf = 1.0 / np.arange(1, len(lexicon) + 1)
    zipf /= zipf.sum()
    endings = ["'s", "'t", "'re", "'ve", "'m", "'ll", "'d"]
    puncts = [".", ",", "!", "?", ";", ":", "-", "(", ")", "\"", "...", "--", "'", "@", "#", "$", "%", "&", "*"]
    seps = [" "] * 40 + ["  ", "   ", "\n", "\n\n", "\t", " \n", "\t\t", "\r\n"]
    out = []
    for _ in range(n_words):
        r = rng.random()
        if r < 0.06:
            out.append(str(int(rng.integers(0, 10 ** int(rng.integers(1, 6))))))
        elif r < 0.12:
            out.append(puncts[int(rng.integers(len(puncts)))])
        else:
            w = lexicon[int(rng.choice(len(lexicon), p=zipf))]
            if rng.random() < 0.1:
                w = w.capitalize()
            if rng.random() < 0.05:
                w += endings[int(rng.integers(len(endings)))]
            out.append(w)
        out.append(seps[int(rng.integers(len(seps)))])
    return "".join(out)


def make_bpe_files(folder: str, seed: int = 3001, vocab_size: int = 2000):
    """vocab.json and merges.txt in GPT-2's format for a byte-level BPE trained
    by the tokenizers package on synthetic_text(seed) (the published GPT-2 files
    are not available).  Returns their paths."""
    import os
    from tokenizers import ByteLevelBPETokenizer
    os.makedirs(folder, exist_ok=True)
    tok = ByteLevelBPETokenizer()
    tok.train_from_iterator([synthetic_text(seed)], vocab_size=vocab_size, min_frequency=2, show_progress=False)
    tok.save_model(folder)
    return os.path.join(folder, "vocab.json"), os.path.join(folder, "merges.txt")
