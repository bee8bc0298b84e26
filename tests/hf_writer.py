"""Write a synthetic model as the Hugging Face files GPT-2 is published as:
model.safetensors (written by the safetensors package's own writer) and
config.json (the keys of GPT-2's published configuration).  Test helper; the
numbers are synth's."""
import json
import os

import numpy as np
import safetensors.numpy as sn


def config_dict(cfg):
    return {"model_type": "gpt2", "activation_function": "gelu_new", "architectures": ["GPT2LMHeadModel"],
            "n_layer": cfg.n_layer, "n_embd": cfg.n_embd, "n_head": cfg.n_head, "n_positions": cfg.n_positions,
            "n_ctx": cfg.n_positions, "vocab_size": cfg.vocab, "n_inner": None,
            "layer_norm_epsilon": cfg.ln_eps, "scale_attn_weights": True,
            "scale_attn_by_inverse_layer_idx": False, "reorder_and_upcast_attn": False,
            "resid_pdrop": 0.1, "embd_pdrop": 0.1, "attn_pdrop": 0.1,
            "bos_token_id": cfg.vocab - 1, "eos_token_id": cfg.vocab - 1,
            "task_specific_params": {"text-generation": {"do_sample": True, "max_length": 50}}}


def write_model(model, folder, prefix="", config_overrides=None, drop=None, replace=None):
    """model.safetensors + config.json in folder; returns their paths.  prefix is
    put before every tensor name; drop removes tensors, replace substitutes arrays
    (both by unprefixed name)."""
    os.makedirs(folder, exist_ok=True)
    tensors = {}
    for name, arr in model.t.items():
        if drop and name in drop:
            continue
        a = replace[name] if replace and name in replace else arr
        tensors[prefix + name] = np.ascontiguousarray(a)
    st = os.path.join(folder, "model.safetensors")
    sn.save_file(tensors, st, metadata={"format": "pt"})
    cfgd = config_dict(model.cfg)
    for k, v in (config_overrides or {}).items():
        if v is ...:
            cfgd.pop(k, None)
        else:
            cfgd[k] = v
    cj = os.path.join(folder, "config.json")
    with open(cj, "w") as f:
        json.dump(cfgd, f, indent=2)
    return st, cj
