"""Write tests/golden/gpt2_124m_fp32_long.json: the oracle's greedy run of the
long-context workload (fp32 GPT-2 124M shape, 8 prompt ids, then greedy decode to
position 1023), for the GPU parity test that cannot afford to run the oracle for
1024 positions itself.

Calls only the oracle (float build) and the seeded input generators.  Stored per
step: the token fed, the oracle's argmax, its top-2 logit margin and max |logit|;
at sampled positions (chunk boundaries of the 64-position attention chunks and the
last position) the logits of the 8 largest ids and of 64 seeded random ids.

  python tests/golden/make_long_context.py
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import Oracle  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gpt2_124m_fp32_long.json")
SAMPLED = [0, 7, 63, 64, 65, 127, 128, 255, 256, 511, 512, 767, 768, 1000, 1023]
N_RANDOM_IDS = 64


def main():
    cfg = synth.CONFIGS[5]
    model = synth.make_model(cfg)
    orc = Oracle(model)
    prompt = [int(t) for t in synth.make_prompt(cfg)]
    rid = np.random.Generator(np.random.PCG64(5005)).choice(cfg.vocab, N_RANDOM_IDS, replace=False)
    toks = list(prompt)
    steps, samples = [], {}
    t0 = time.time()
    for pos in range(cfg.n_steps):
        am, lg = orc.step(toks[pos], pos)
        lg = np.asarray(lg, np.float64)
        part = np.partition(lg, -2)
        steps.append({"tok": toks[pos], "argmax": int(am), "margin": float(part[-1] - part[-2]),
                      "maxabs": float(np.abs(lg).max())})
        if pos in SAMPLED:
            top = np.argsort(-lg, kind="stable")[:8]
            ids = [int(i) for i in top] + [int(i) for i in rid]
            samples[str(pos)] = {"ids": ids, "logits": [float(lg[i]) for i in ids]}
        if pos + 1 >= len(toks) and pos + 1 < cfg.n_steps:
            toks.append(int(am))
        if pos % 128 == 0:
            print(f"pos {pos}  {time.time() - t0:.1f} s", flush=True)
    orc.close()
    doc = {
        "what": "oracle (float build) greedy run of the long-context workload: fp32 GPT-2 124M "
                "shape, weight seed 1002, prompt seed 2005, 8 prompt ids then greedy to position 1023",
        "written_by": "tests/golden/make_long_context.py (oracle and synth only)",
        "n_prompt": cfg.n_prompt, "n_steps": cfg.n_steps, "prompt": prompt,
        "steps": steps, "samples": samples,
    }
    with open(OUT, "w") as f:
        json.dump(doc, f, separators=(",", ":"))
    print(f"wrote {OUT} ({os.path.getsize(OUT)} bytes) in {time.time() - t0:.1f} s")


if __name__ == "__main__":
    main()
