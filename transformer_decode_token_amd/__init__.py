"""Python binding of libgpt2dec.so, the MI355X batch-1 GPT-2 decode library.

Argument marshalling only: every step of the forward pass runs in the HIP
kernels behind the C ABI (include/gpt2dec.h).  The functions carry the C names.
There is no fallback: if the library is not built, or no GPU is present, the
calls fail with an error.
"""
import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgpt2dec.so")

GPT2_OK, GPT2_E_INVAL, GPT2_E_NOMEM, GPT2_E_DEVICE, GPT2_E_STATE, GPT2_E_NUMERIC = 0, -1, -2, -3, -4, -5
GPT2_W_FP32, GPT2_W_FP16, GPT2_W_INT4 = 0, 1, 2
WDTYPES = {"fp32": GPT2_W_FP32, "fp16": GPT2_W_FP16, "int4": GPT2_W_INT4}
ERROR_NAMES = {GPT2_E_INVAL: "GPT2_E_INVAL", GPT2_E_NOMEM: "GPT2_E_NOMEM",
               GPT2_E_DEVICE: "GPT2_E_DEVICE", GPT2_E_STATE: "GPT2_E_STATE",
               GPT2_E_NUMERIC: "GPT2_E_NUMERIC"}

# the symbols include/gpt2dec.h declares
ABI_FUNCTIONS = ("gpt2_load", "gpt2_load_safetensors", "gpt2_get_config", "gpt2_set_stream",
                 "gpt2_prefill", "gpt2_step", "gpt2_generate", "gpt2_generate_noalloc", "gpt2_generate_sample",
                 "gpt2_reset", "gpt2_free", "gpt2_last_error", "gpt2_filled",
                 "gpt2_debug_dequant", "gpt2_debug_fill_kv", "gpt2_debug_geometry", "gpt2_debug_trace",
                 "gpt2_tokenizer_load", "gpt2_tokenize", "gpt2_detokenize", "gpt2_tokenizer_free")


class Gpt2Error(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {message}")
        self.code = code


class gpt2_config(C.Structure):
    _fields_ = [("n_layer", C.c_int), ("n_embd", C.c_int), ("n_head", C.c_int),
                ("n_positions", C.c_int), ("vocab_size", C.c_int), ("ln_eps", C.c_float),
                ("wdtype", C.c_int), ("q4_group", C.c_int)]


_PP = C.POINTER(C.c_void_p)


class gpt2_weights(C.Structure):
    _fields_ = [("wte", C.c_void_p), ("wpe", C.c_void_p),
                ("ln1_w", _PP), ("ln1_b", _PP), ("c_attn_w", _PP), ("c_attn_b", _PP),
                ("attn_proj_w", _PP), ("attn_proj_b", _PP), ("ln2_w", _PP), ("ln2_b", _PP),
                ("c_fc_w", _PP), ("c_fc_b", _PP), ("mlp_proj_w", _PP), ("mlp_proj_b", _PP),
                ("lnf_w", C.c_void_p), ("lnf_b", C.c_void_p)]


_lib = None


def lib():
    """The loaded libgpt2dec.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run python -m transformer_decode_token_amd.build")
        L = C.CDLL(LIB_PATH)
        L.gpt2_load.argtypes = [C.POINTER(gpt2_config), C.POINTER(gpt2_weights), C.POINTER(C.c_void_p)]
        L.gpt2_load_safetensors.argtypes = [C.c_char_p, C.c_char_p, C.c_int, C.POINTER(C.c_void_p)]
        L.gpt2_get_config.argtypes = [C.c_void_p, C.POINTER(gpt2_config)]
        L.gpt2_set_stream.argtypes = [C.c_void_p, C.c_void_p]
        L.gpt2_step.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.POINTER(C.c_int)]
        L.gpt2_generate.argtypes = [C.c_void_p, C.POINTER(C.c_int), C.c_int, C.c_int, C.POINTER(C.c_int)]
        L.gpt2_prefill.argtypes = [C.c_void_p, C.POINTER(C.c_int), C.c_int, C.c_void_p, C.POINTER(C.c_int)]
        L.gpt2_generate_noalloc.argtypes = [C.c_void_p, C.POINTER(C.c_int), C.c_int, C.c_int, C.POINTER(C.c_int)]
        L.gpt2_generate_sample.argtypes = [C.c_void_p, C.POINTER(C.c_int), C.c_int, C.c_int, C.c_float,
                                           C.c_ulonglong, C.POINTER(C.c_int)]
        L.gpt2_reset.argtypes = [C.c_void_p]
        L.gpt2_free.argtypes = [C.c_void_p]
        L.gpt2_free.restype = None
        L.gpt2_last_error.argtypes = [C.c_void_p]
        L.gpt2_last_error.restype = C.c_char_p
        L.gpt2_filled.argtypes = [C.c_void_p]
        L.gpt2_debug_dequant.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_void_p]
        L.gpt2_debug_fill_kv.argtypes = [C.c_void_p, C.c_float]
        L.gpt2_debug_geometry.argtypes = [C.c_void_p, C.POINTER(C.c_int), C.POINTER(C.c_int)]
        L.gpt2_debug_trace.argtypes = [C.c_void_p, C.c_int, C.c_void_p, C.c_longlong,
                                       C.POINTER(C.c_int)]
        L.gpt2_tokenizer_load.argtypes = [C.c_char_p, C.c_char_p, C.POINTER(C.c_void_p)]
        L.gpt2_tokenize.argtypes = [C.c_void_p, C.c_char_p, C.c_size_t, C.c_void_p, C.c_int, C.POINTER(C.c_int)]
        L.gpt2_detokenize.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_char_p, C.c_size_t,
                                      C.POINTER(C.c_size_t)]
        L.gpt2_tokenizer_free.argtypes = [C.c_void_p]
        L.gpt2_tokenizer_free.restype = None
        _lib = L
    return _lib


def _check(rc, ctx):
    if rc != GPT2_OK:
        msg = lib().gpt2_last_error(ctx)
        raise Gpt2Error(rc, msg.decode() if msg else "")


class Context:
    """Owns one gpt2_ctx*; freed with gpt2_free."""

    def __init__(self, handle, cfg):
        self.handle = handle
        self.cfg = cfg

    def close(self):
        if self.handle:
            lib().gpt2_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


HF_BLOCK = ("ln_1.weight", "ln_1.bias", "attn.c_attn.weight", "attn.c_attn.bias",
            "attn.c_proj.weight", "attn.c_proj.bias", "ln_2.weight", "ln_2.bias",
            "mlp.c_fc.weight", "mlp.c_fc.bias", "mlp.c_proj.weight", "mlp.c_proj.bias")
_FIELDS = ("ln1_w", "ln1_b", "c_attn_w", "c_attn_b", "attn_proj_w", "attn_proj_b", "ln2_w",
           "ln2_b", "c_fc_w", "c_fc_b", "mlp_proj_w", "mlp_proj_b")


def gpt2_load(n_layer, n_embd, n_head, n_positions, vocab_size, tensors, wdtype="fp32",
              ln_eps=1e-5, q4_group=32):
    """tensors: mapping of Hugging Face names (without the 'transformer.' prefix) to host
    float32 arrays in the checkpoint layout.  Returns a Context."""
    cfg = gpt2_config(n_layer, n_embd, n_head, n_positions, vocab_size, ln_eps,
                      WDTYPES[wdtype] if isinstance(wdtype, str) else int(wdtype), q4_group)
    keep = {}

    def arr(name):
        a = np.ascontiguousarray(tensors[name], dtype=np.float32)
        keep[name] = a
        return a.ctypes.data

    w = gpt2_weights()
    w.wte, w.wpe = arr("wte.weight"), arr("wpe.weight")
    lists = {}
    for f, n in zip(_FIELDS, HF_BLOCK):
        lists[f] = (C.c_void_p * n_layer)(*[arr(f"h.{l}.{n}") for l in range(n_layer)])
        setattr(w, f, C.cast(lists[f], _PP))
    w.lnf_w, w.lnf_b = arr("ln_f.weight"), arr("ln_f.bias")
    h = C.c_void_p()
    rc = lib().gpt2_load(C.byref(cfg), C.byref(w), C.byref(h))
    _check(rc, None)
    return Context(h, cfg)


def gpt2_load_safetensors(safetensors_path, config_path, wdtype="fp32"):
    """Load from a Hugging Face model.safetensors and its config.json, as published."""
    h = C.c_void_p()
    rc = lib().gpt2_load_safetensors(os.fsencode(safetensors_path), os.fsencode(config_path),
                                     WDTYPES[wdtype] if isinstance(wdtype, str) else int(wdtype), C.byref(h))
    _check(rc, None)
    cfg = gpt2_config()
    _check(lib().gpt2_get_config(h, C.byref(cfg)), h)
    return Context(h, cfg)


def gpt2_get_config(ctx):
    cfg = gpt2_config()
    _check(lib().gpt2_get_config(ctx.handle, C.byref(cfg)), ctx.handle)
    return cfg


def gpt2_set_stream(ctx, hip_stream):
    _check(lib().gpt2_set_stream(ctx.handle, C.c_void_p(hip_stream or 0)), ctx.handle)


def gpt2_step(ctx, token_id, position, want_logits=True):
    """Returns (argmax_id, logits float32[V] or None)."""
    logits = np.empty(ctx.cfg.vocab_size, np.float32) if want_logits else None
    am = C.c_int(-1)
    rc = lib().gpt2_step(ctx.handle, int(token_id), int(position),
                         logits.ctypes.data if want_logits else None, C.byref(am))
    _check(rc, ctx.handle)
    return am.value, logits


def gpt2_generate(ctx, prompt, n_new):
    p = np.ascontiguousarray(prompt, np.int32)
    out = np.empty(int(n_new), np.int32)
    rc = lib().gpt2_generate(ctx.handle, p.ctypes.data_as(C.POINTER(C.c_int)), p.size, int(n_new),
                             out.ctypes.data_as(C.POINTER(C.c_int)))
    _check(rc, ctx.handle)
    return out


def gpt2_prefill(ctx, tokens, want_logits=True):
    """The ids at positions filled .. filled + len(tokens) - 1 through every layer in one call
    (their cache rows appended); returns (argmax of the last position, its logits or None)."""
    t = np.ascontiguousarray(tokens, np.int32)
    logits = np.empty(ctx.cfg.vocab_size, np.float32) if want_logits else None
    am = C.c_int(-1)
    rc = lib().gpt2_prefill(ctx.handle, t.ctypes.data_as(C.POINTER(C.c_int)), t.size,
                            logits.ctypes.data if want_logits else None, C.byref(am))
    _check(rc, ctx.handle)
    return am.value, logits


def gpt2_generate_noalloc(ctx, prompt, n_new):
    p = np.ascontiguousarray(prompt, np.int32)
    out = np.empty(int(n_new), np.int32)
    rc = lib().gpt2_generate_noalloc(ctx.handle, p.ctypes.data_as(C.POINTER(C.c_int)), p.size, int(n_new),
                                     out.ctypes.data_as(C.POINTER(C.c_int)))
    _check(rc, ctx.handle)
    return out


def gpt2_generate_sample(ctx, prompt, n_new, temperature, seed):
    p = np.ascontiguousarray(prompt, np.int32)
    out = np.empty(int(n_new), np.int32)
    rc = lib().gpt2_generate_sample(ctx.handle, p.ctypes.data_as(C.POINTER(C.c_int)), p.size, int(n_new),
                                    float(temperature), int(seed), out.ctypes.data_as(C.POINTER(C.c_int)))
    _check(rc, ctx.handle)
    return out


def gpt2_reset(ctx):
    _check(lib().gpt2_reset(ctx.handle), ctx.handle)


def gpt2_free(ctx):
    ctx.close()


def gpt2_last_error(ctx=None):
    m = lib().gpt2_last_error(ctx.handle if ctx is not None else None)
    return m.decode() if m else ""


def gpt2_filled(ctx):
    return lib().gpt2_filled(ctx.handle)


def gpt2_debug_dequant(ctx, layer, which):
    E, V = ctx.cfg.n_embd, ctx.cfg.vocab_size
    F = 4 * E
    shape = {0: (3 * E, E), 1: (E, E), 2: (F, E), 3: (E, F), 4: (V, E)}[which]
    out = np.empty(shape, np.float32)
    _check(lib().gpt2_debug_dequant(ctx.handle, int(layer), int(which), out.ctypes.data), ctx.handle)
    return out


def gpt2_debug_fill_kv(ctx, value):
    _check(lib().gpt2_debug_fill_kv(ctx.handle, float(value)), ctx.handle)


def gpt2_debug_geometry(ctx):
    g, t = C.c_int(), C.c_int()
    _check(lib().gpt2_debug_geometry(ctx.handle, C.byref(g), C.byref(t)), ctx.handle)
    return g.value, t.value


def gpt2_debug_trace(ctx, steps, fetch=False):
    """Record `steps` steps of every later run (-1: leave the setting as it is); with
    fetch=True, first return the last run's record as int64 [recorded steps][5L+1][G][4]
    (None if nothing is recorded)."""
    out = None
    if fetch:
        rec = C.c_int(0)
        _check(lib().gpt2_debug_trace(ctx.handle, -1, None, 0, C.byref(rec)), ctx.handle)
        if rec.value > 0:
            g, _ = gpt2_debug_geometry(ctx)
            out = np.zeros((rec.value, 5 * ctx.cfg.n_layer + 1, g, 4), np.int64)
            _check(lib().gpt2_debug_trace(ctx.handle, -1, out.ctypes.data, out.size, None), ctx.handle)
    _check(lib().gpt2_debug_trace(ctx.handle, int(steps), None, 0, None), ctx.handle)
    return out


class Tokenizer:
    """Owns one gpt2_tokenizer*; freed with gpt2_tokenizer_free."""

    def __init__(self, handle):
        self.handle = handle

    def close(self):
        if self.handle:
            lib().gpt2_tokenizer_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gpt2_tokenizer_load(vocab_json_path, merges_txt_path):
    h = C.c_void_p()
    _check(lib().gpt2_tokenizer_load(os.fsencode(vocab_json_path), os.fsencode(merges_txt_path), C.byref(h)), None)
    return Tokenizer(h)


def gpt2_tokenize(tok, text):
    """Token ids (int32 array) of a str (encoded UTF-8) or bytes."""
    data = text.encode("utf-8") if isinstance(text, str) else bytes(text)
    n = C.c_int(0)
    _check(lib().gpt2_tokenize(tok.handle, data, len(data), None, 0, C.byref(n)), None)
    out = np.empty(n.value, np.int32)
    _check(lib().gpt2_tokenize(tok.handle, data, len(data), out.ctypes.data, out.size, C.byref(n)), None)
    return out


def gpt2_detokenize(tok, ids):
    """The bytes of the ids."""
    ids = np.ascontiguousarray(ids, np.int32)
    m = C.c_size_t(0)
    _check(lib().gpt2_detokenize(tok.handle, ids.ctypes.data, ids.size, None, 0, C.byref(m)), None)
    buf = C.create_string_buffer(max(m.value, 1))
    _check(lib().gpt2_detokenize(tok.handle, ids.ctypes.data, ids.size, buf, m.value, C.byref(m)), None)
    return buf.raw[:m.value]
