"""Write the stored expected values under tests/golden/ -- calls only the oracle.

    python tests/golden/make_golden.py

tiny_dense_fp32_greedy.json: the oracle's greedy stream on the tiny dense fp32
workload (hidden 64, 2 layers, 4 q / 2 kv heads, head_dim 16, inter 256, vocab
512, seed 0; 16-token prompt, 16 greedy steps, fp32 cache).  The reference
pages print no logits or token streams for any model, so this file is a
regression fixture of the pinned oracle, not a value taken from the pages.
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402


def main():
    cfg = synth.TINY
    dec = oracle.Decoder.from_synth(cfg)
    pr = synth.prompt(cfg)
    toks, lg = dec.generate(pr, cfg.n_decode)
    gaps = []
    for l in lg:
        s = np.sort(l)
        gaps.append(float(s[-1] - s[-2]))
    out = {
        "config": cfg.name,
        "source": "oracle (liboracle fp64), tests/golden/make_golden.py",
        "prompt": [int(t) for t in pr],
        "tokens": [int(t) for t in toks],
        "top_logit": [float(np.max(l)) for l in lg],
        "top2_gap": gaps,
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_dense_fp32_greedy.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(path)


if __name__ == "__main__":
    main()
