"""Independent reference for the oracle: Hugging Face transformers' GPT2LMHeadModel.

The gpt2.s README ("Verify") checks the program against Hugging Face GPT-2 in
PyTorch; here the same library implementation (built from a config, no
download) is loaded with the synthetic weights and run in float64 over the
whole sequence with its own causal mask.  It shares nothing with the oracle.
"""
import numpy as np
import torch


def hf_model(model, dtype=torch.float64):
    from transformers import GPT2Config, GPT2LMHeadModel
    c = model.cfg
    hc = GPT2Config(n_layer=c.n_layer, n_embd=c.n_embd, n_head=c.n_head,
                    n_positions=c.n_positions, vocab_size=c.vocab,
                    activation_function="gelu_new",
                    # the oracle and the library carry eps as a float32 value
                    layer_norm_epsilon=float(np.float32(c.ln_eps)),
                    resid_pdrop=0.0, embd_pdrop=0.0, attn_pdrop=0.0,
                    scale_attn_weights=True, scale_attn_by_inverse_layer_idx=False,
                    reorder_and_upcast_attn=False, bos_token_id=0, eos_token_id=0,
                    tie_word_embeddings=True)
    hc._attn_implementation = "eager"
    m = GPT2LMHeadModel(hc)
    sd = {}
    for name, arr in model.t.items():
        sd["transformer." + name] = torch.from_numpy(np.asarray(arr, np.float32).copy())
    missing, unexpected = m.load_state_dict(sd, strict=False)
    assert not unexpected, unexpected
    # only buffers (attention masks) and the tied lm_head may be absent
    assert all(k.endswith(".attn.bias") or k.endswith(".attn.masked_bias") or k == "lm_head.weight"
               for k in missing), missing
    m.tie_weights()
    assert m.lm_head.weight.data_ptr() == m.transformer.wte.weight.data_ptr()
    return m.to(dtype).eval()


@torch.no_grad()
def hf_logits(m, tokens, dtype=torch.float64):
    """Logits [n][V] for every position of the token sequence."""
    ids = torch.as_tensor(np.asarray(tokens, np.int64))[None, :]
    out = m(input_ids=ids, use_cache=False)
    return out.logits[0].to(dtype).numpy()
