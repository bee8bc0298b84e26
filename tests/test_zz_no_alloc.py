"""gpt2_generate_noalloc, the entry point that allocates nothing (its working
words in the library's static device array), against gpt2_generate on the same
model: identical ids and bit-identical logits of the next pass, on two calls in
a row, the second with a smaller input; and a model too large for the array is
refused before any device work."""
import ctypes as C

import numpy as np
import pytest

import synth
import transformer_decode_token_amd as g2
from tests.gpu_util import load_gpu

pytestmark = pytest.mark.gpu


def _tiny_rich():
    return synth.variant(synth.CONFIGS[1], init="small", weight_seed=1101, name="tiny-rich")


@pytest.mark.parametrize("cfg", [_tiny_rich(), synth.CONFIGS[2], synth.CONFIGS[3]], ids=lambda c: c.name)
def test_noalloc_matches_generate(cfg):
    model = synth.make_model(cfg)
    prompt = synth.make_prompt(cfg)
    ref, na = load_gpu(model), load_gpu(model)
    for n_prompt, n_new in ((len(prompt), 20), (3, 5)):   # the second call: a smaller input
        p = np.asarray(prompt[:n_prompt], np.int32)
        g2.gpt2_reset(ref)
        g2.gpt2_reset(na)
        want = g2.gpt2_generate(ref, p, n_new)
        # through the C ABI directly
        got = np.empty(n_new, np.int32)
        rc = g2.lib().gpt2_generate_noalloc(na.handle, p.ctypes.data_as(C.POINTER(C.c_int)), p.size, n_new,
                                            got.ctypes.data_as(C.POINTER(C.c_int)))
        assert rc == g2.GPT2_OK, g2.gpt2_last_error(na)
        assert np.array_equal(got, want), (n_prompt, n_new)
        assert g2.gpt2_filled(na) == g2.gpt2_filled(ref) == n_prompt + n_new - 1
        # the cache rows it left: the next pass reads them all
        pos = n_prompt + n_new - 1
        _, l_ref = g2.gpt2_step(ref, int(want[-1]), pos)
        _, l_na = g2.gpt2_step(na, int(want[-1]), pos)
        assert np.array_equal(l_ref, l_na), (n_prompt, n_new)
    ref.close()
    na.close()


def test_noalloc_refuses_a_model_beyond_the_array():
    # 200 layers of the tiny shape need about 18 MB of working words (> 16 MiB)
    cfg = synth.variant(_tiny_rich(), n_layer=200, name="tiny-200")
    ctx = load_gpu(synth.make_model(cfg))
    with pytest.raises(g2.Gpt2Error) as e:
        g2.gpt2_generate_noalloc(ctx, [1, 2, 3], 2)
    assert e.value.code == g2.GPT2_E_INVAL
    assert "static scratch" in g2.gpt2_last_error(ctx)
    assert g2.gpt2_filled(ctx) == 0
    ctx.close()
