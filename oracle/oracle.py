"""ctypes wrapper of the C oracle (TEST INFRASTRUCTURE ONLY; see gpt2_oracle.c)."""
import ctypes as C
import os

import numpy as np

from . import build_oracle

_LIBS = {}


class OracleLib:
    """One build of the oracle: kind 'f32' (float) or 'f64' (double)."""

    def __init__(self, kind: str = "f32"):
        path = build_oracle.lib_path(kind)
        if not os.path.exists(path):
            build_oracle.build()
        self.kind = kind
        self.lib = C.CDLL(path)
        self.real = np.float32 if kind == "f32" else np.float64
        assert self.lib.oracle_real_bytes() == np.dtype(self.real).itemsize
        rp = np.ctypeslib.ndpointer(self.real, flags="C_CONTIGUOUS")
        L = self.lib
        L.oracle_n_tensors.argtypes = [C.c_int]
        L.oracle_n_tensors.restype = C.c_int
        L.oracle_new.argtypes = [C.POINTER(C.c_int), C.c_float, C.c_int, C.c_int,
                                 C.POINTER(C.c_void_p)]
        L.oracle_new.restype = C.c_void_p
        L.oracle_free.argtypes = [C.c_void_p]
        L.oracle_reset.argtypes = [C.c_void_p]
        L.oracle_step.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_void_p]
        L.oracle_step.restype = C.c_int
        L.oracle_prefill_last.argtypes = [C.c_void_p, C.POINTER(C.c_int), C.c_int, C.c_void_p]
        L.oracle_prefill_last.restype = C.c_int
        L.oracle_get_weight.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_void_p]
        L.oracle_get_weight.restype = C.c_long
        L.oracle_poison_cache_after.argtypes = [C.c_void_p, C.c_int, C.c_float]
        L.oracle_layernorm.argtypes = [rp, rp, rp, C.c_int, self._rt(), rp]
        L.oracle_gelu_new.argtypes = [self._rt()]
        L.oracle_gelu_new.restype = self._rt()
        L.oracle_linear_conv1d.argtypes = [rp, rp, C.c_void_p, C.c_int, C.c_int, rp]
        L.oracle_attn_head.argtypes = [rp, rp, rp, C.c_int, C.c_int, C.c_int, C.c_void_p, rp]
        L.oracle_f32_to_f16.argtypes = [C.c_float]
        L.oracle_f32_to_f16.restype = C.c_uint16
        L.oracle_f16_to_f32.argtypes = [C.c_uint16]
        L.oracle_f16_to_f32.restype = C.c_float
        f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
        u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
        L.oracle_q4_group.argtypes = [f32p, C.c_int, u8p, C.POINTER(C.c_float),
                                      C.POINTER(C.c_float), f32p]
        L.oracle_argmax.argtypes = [rp, C.c_int]
        L.oracle_argmax.restype = C.c_int
        L.oracle_xorshift64s.argtypes = [C.POINTER(C.c_uint64)]
        L.oracle_xorshift64s.restype = C.c_uint64
        L.oracle_uniform.argtypes = [C.POINTER(C.c_uint64)]
        L.oracle_uniform.restype = C.c_float
        L.oracle_sample.argtypes = [rp, C.c_int, self._rt(), self._rt()]
        L.oracle_sample.restype = C.c_int

    def _rt(self):
        return C.c_float if self.kind == "f32" else C.c_double

    # ---- primitives ------------------------------------------------------
    def layernorm(self, x, g, b, eps):
        x, g, b = (np.ascontiguousarray(a, self.real) for a in (x, g, b))
        y = np.empty_like(x)
        self.lib.oracle_layernorm(x, g, b, x.size, eps, y)
        return y

    def gelu_new(self, x):
        return np.array([self.lib.oracle_gelu_new(float(v)) for v in np.ravel(x)], self.real)

    def linear_conv1d(self, x, W, b=None):
        x = np.ascontiguousarray(x, self.real)
        W = np.ascontiguousarray(W, self.real)
        K, N = W.shape
        y = np.empty(N, self.real)
        bp = None
        if b is not None:
            b = np.ascontiguousarray(b, self.real)
            bp = b.ctypes.data_as(C.c_void_p)
        self.lib.oracle_linear_conv1d(x, W, bp, K, N, y)
        return y

    def attn_head(self, q, Kc, Vc, pos):
        """q[D]; Kc, Vc [T][D] with T > pos. Returns (out[D], probs[pos+1])."""
        q = np.ascontiguousarray(q, self.real)
        Kc = np.ascontiguousarray(Kc, self.real)
        Vc = np.ascontiguousarray(Vc, self.real)
        D = q.size
        probs = np.empty(pos + 1, self.real)
        out = np.empty(D, self.real)
        self.lib.oracle_attn_head(q, Kc, Vc, pos, Kc.shape[1], D,
                                  probs.ctypes.data_as(C.c_void_p), out)
        return out, probs

    def f32_to_f16_bits(self, arr):
        return np.array([self.lib.oracle_f32_to_f16(float(v)) for v in np.ravel(arr)],
                        np.uint16)

    def f16_bits_to_f32(self, bits):
        return np.array([self.lib.oracle_f16_to_f32(int(v)) for v in np.ravel(bits)],
                        np.float32)

    def q4_group(self, w):
        w = np.ascontiguousarray(w, np.float32)
        q = np.empty(w.size, np.uint8)
        deq = np.empty(w.size, np.float32)
        s = C.c_float()
        mn = C.c_float()
        self.lib.oracle_q4_group(w, w.size, q, C.byref(s), C.byref(mn), deq)
        return q, np.float32(s.value), np.float32(mn.value), deq

    def argmax(self, v):
        v = np.ascontiguousarray(v, self.real)
        return self.lib.oracle_argmax(v, v.size)

    def xorshift64s(self, seed, n):
        """n successive xorshift64* outputs from state `seed`; returns (outputs, state)."""
        st = C.c_uint64(seed)
        out = np.array([self.lib.oracle_xorshift64s(C.byref(st)) for _ in range(n)], np.uint64)
        return out, st.value

    def uniforms(self, seed, n):
        st = C.c_uint64(seed)
        return np.array([self.lib.oracle_uniform(C.byref(st)) for _ in range(n)], np.float32)

    def sample(self, logits, temperature, u):
        logits = np.ascontiguousarray(logits, self.real)
        return self.lib.oracle_sample(logits, logits.size, temperature, u)


def load_lib(kind: str = "f32") -> OracleLib:
    if kind not in _LIBS:
        _LIBS[kind] = OracleLib(kind)
    return _LIBS[kind]


WDTYPES = {"fp32": 0, "fp16": 1, "int4": 2}


class Oracle:
    """A whole oracle model built from a synth.Model (host fp32 arrays, HF layout)."""

    def __init__(self, model, kind: str = "f32"):
        self.L = load_lib(kind)
        self.model = model
        c = model.cfg
        self.V = c.vocab
        shape = (C.c_int * 5)(c.n_layer, c.n_embd, c.n_head, c.n_positions, c.vocab)
        tensors = model.flat_tensors()
        assert len(tensors) == self.L.lib.oracle_n_tensors(c.n_layer)
        self._keep = [np.ascontiguousarray(t, np.float32) for t in tensors]
        ptrs = (C.c_void_p * len(self._keep))(*[t.ctypes.data for t in self._keep])
        h = self.L.lib.oracle_new(shape, C.c_float(c.ln_eps), WDTYPES[c.wdtype], c.q4_group,
                                  ptrs)
        self._keep = None  # the oracle copied everything
        if not h:
            raise ValueError("oracle rejected the configuration")
        self.h = h

    def close(self):
        if self.h:
            self.L.lib.oracle_free(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reset(self):
        self.L.lib.oracle_reset(self.h)

    def step(self, token, position, want_logits=True):
        logits = np.empty(self.V, self.L.real) if want_logits else None
        ptr = logits.ctypes.data_as(C.c_void_p) if want_logits else None
        am = self.L.lib.oracle_step(self.h, int(token), int(position), ptr)
        if am < 0:
            raise ValueError(f"oracle_step rejected token={token} position={position}")
        return am, logits

    def prefill_last(self, toks):
        toks = np.ascontiguousarray(toks, np.int32)
        logits = np.empty(self.V, self.L.real)
        am = self.L.lib.oracle_prefill_last(
            self.h, toks.ctypes.data_as(C.POINTER(C.c_int)), toks.size,
            logits.ctypes.data_as(C.c_void_p))
        if am < 0:
            raise ValueError("oracle_prefill_last rejected the input")
        return am, logits

    def weight(self, layer, which):
        c = self.model.cfg
        E, F, V = c.n_embd, 4 * c.n_embd, c.vocab
        n = {0: 3 * E * E, 1: E * E, 2: F * E, 3: E * F, 4: V * E}[which]
        out = np.empty(n, np.float32)
        got = self.L.lib.oracle_get_weight(self.h, layer, which, out.ctypes.data_as(C.c_void_p))
        assert got == n
        return out

    def poison_cache_after(self, position, value):
        self.L.lib.oracle_poison_cache_after(self.h, int(position), C.c_float(value))
