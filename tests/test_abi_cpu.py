"""The C-ABI library on a machine without a GPU: it loads, exports every symbol
include/gpt2dec.h declares, validates arguments before touching a device, and
reports the missing device as GPT2_E_DEVICE (no CPU fallback)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import synth
import transformer_decode_token_amd as g2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(g2.LIB_PATH):
        from transformer_decode_token_amd import build
        build.build()
    return g2.lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "gpt2dec.h")).read()
    return re.findall(r"GPT2DEC_API\s+[\w\s\*]*?\b(gpt2_\w+)\s*\(", text)


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert sorted(names) == sorted(g2.ABI_FUNCTIONS)
    for n in names:
        assert hasattr(lib, n), n
    out = os.popen(f"nm -D --defined-only {g2.LIB_PATH}").read()
    exported = set(re.findall(r"\bT (gpt2_\w+)", out))
    assert set(names) <= exported


def _cpu_has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def test_invalid_configs_rejected_before_device(lib):
    m = synth.make_model(1)
    c = m.cfg
    bad = [dict(n_head=3),                       # 128 not divisible by 3
           dict(n_embd=256, n_head=4),           # shape not built
           dict(n_layer=0)]
    for kw in bad:
        args = dict(n_layer=c.n_layer, n_embd=c.n_embd, n_head=c.n_head,
                    n_positions=c.n_positions, vocab_size=c.vocab)
        args.update(kw)
        with pytest.raises((g2.Gpt2Error, KeyError)) as e:
            g2.gpt2_load(args["n_layer"], args["n_embd"], args["n_head"], args["n_positions"],
                         args["vocab_size"], m.t)
        if isinstance(e.value, g2.Gpt2Error):
            assert e.value.code == g2.GPT2_E_INVAL
            assert g2.gpt2_last_error()
    with pytest.raises(g2.Gpt2Error) as e:
        g2.gpt2_load(c.n_layer, c.n_embd, c.n_head, c.n_positions, c.vocab, m.t, wdtype="int4",
                     q4_group=16)
    assert e.value.code == g2.GPT2_E_INVAL


def test_null_arguments(lib):
    assert lib.gpt2_load(None, None, None) == g2.GPT2_E_INVAL
    h = C.c_void_p()
    assert lib.gpt2_load(None, None, C.byref(h)) == g2.GPT2_E_INVAL
    assert not h.value
    assert lib.gpt2_step(None, 0, 0, None, None) == g2.GPT2_E_INVAL
    assert lib.gpt2_reset(None) == g2.GPT2_E_INVAL
    assert lib.gpt2_generate_sample(None, None, 0, 0, 0.8, 1, None) == g2.GPT2_E_INVAL
    assert lib.gpt2_filled(None) == -1
    lib.gpt2_free(None)


@pytest.mark.skipif(_cpu_has_gpu(), reason="checks the no-GPU path")
def test_no_device_is_an_error_not_a_fallback(lib):
    m = synth.make_model(1)
    c = m.cfg
    with pytest.raises(g2.Gpt2Error) as e:
        g2.gpt2_load(c.n_layer, c.n_embd, c.n_head, c.n_positions, c.vocab, m.t)
    assert e.value.code == g2.GPT2_E_DEVICE
    assert "device" in g2.gpt2_last_error().lower()
