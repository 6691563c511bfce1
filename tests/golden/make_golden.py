"""Writes tests/golden/tiny_greedy.json from the CPU oracle alone.

Workload: the tiny decoder (2 layers, hidden 256, 4 q / 2 kv heads of 64, SwiGLU
1024, vocab 1024, float32, weights N(0, 0.02) from seed 0), a 64-token prompt
uniform in [0, 1024) from seed 1, prefilled token by token, then 8 greedy decode
steps.  The stored tokens and top-2 margins are a regression pin of the oracle;
nothing here comes from the GPU path.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402


def tiny_greedy(steps: int = 8, prompt_len: int = 64):
    cfg = synth.TINY
    model = oracle.Model(cfg, synth.make_weights(cfg))
    prompt = synth.prompt_tokens(cfg, 1, prompt_len)
    kc, vc = model.new_cache(1, prompt_len + steps + 8)
    sl = np.zeros(1, np.int32)
    logits, tok = model.prefill(prompt, kc, vc, sl)
    tokens, margins, sums = [], [], []
    for _ in range(steps):
        tokens.append(int(tok[0]))
        top = np.sort(logits[0].astype(np.float32))[-2:]
        margins.append(float(top[1] - top[0]))
        logits, tok = model.step(tok, kc, vc, sl)
        sums.append(float(logits[0].sum()))
    return {"prompt_len": prompt_len, "steps": steps, "greedy_tokens": tokens,
            "top2_margins_f32": margins, "logit_sums_after_each_step": sums}


if __name__ == "__main__":
    out = tiny_greedy()
    out["source"] = "tests/golden/make_golden.py (oracle only)"
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_greedy.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(path, out["greedy_tokens"])
