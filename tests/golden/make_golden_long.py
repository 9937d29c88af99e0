"""Write the long-prompt expected values under tests/golden/ -- calls only the
oracle (and the seeded input generators of ``synth``).

    python tests/golden/make_golden_long.py [k2h_bf16_p512] [k2h_i8_p1024] [k2h_fp8_w2_p300] ...

Each file holds the oracle's greedy run of the full-depth 3.7B-shaped model
(hidden 2560, 36 layers, 32 q / 8 kv heads, head_dim 128, SwiGLU 10240, vocab
250624, seeded bf16 weights) on the seeded uniform prompt, position by
position from position 0, then 4 decode steps fed with the oracle's own
argmax:

  k2h_bf16_p512.npz   bf16 KV cache, context 4096, 512-token prompt
                      (the decode positions then have prefix lengths
                      513..516)
  k2h_i8_p1024.npz    int8 KV cache, context 32768, 1024-token prompt, so
                      the cache the decode steps read is the one a real
                      prefill wrote (no synthetic history)

  k2h_{fp8,mxfp4,q4s}_w2_p300.npz
                      the quantized-weight models (fp8 E4M3 + row scale,
                      MXFP4, Q4S; int8 KV) at their full widths but two
                      layers and a 4096-token vocabulary, 300-token prompt
                      (the prefill's 256 + 44 chunks at the real product
                      shapes, with an oracle run of minutes)

Arrays: ``prompt`` (int32), ``tokens`` (int32 [5]: the argmax after the last
prompt position and after each decode step), ``logits`` (float32 [5][vocab],
the oracle's fp64 logits rounded to fp32), ``top2_gap`` (float64 [5]).  The
pages print no logits for any model: these are regression fixtures of the
pinned oracle, not values taken from the pages.  Each run takes tens of
minutes of CPU time (fp64, OpenMP over rows).
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
N_EMIT = 5

def _w2(name: str):
    return synth.CONFIGS[name].replace(n_layers=2, vocab=4096, cap=512)


RUNS = {
    "k2h_bf16_p512": (synth.K2H_BF16, 512),
    "k2h_i8_p1024": (synth.K2H_BF16_I8_LONG, 1024),
    "k2h_fp8_w2_p300": (_w2("k2h-3.7b-fp8-kvi8-ctx4096"), 300),
    "k2h_mxfp4_w2_p300": (_w2("k2h-3.7b-mxfp4-kvi8-ctx4096"), 300),
    "k2h_q4s_w2_p300": (_w2("k2h-3.7b-q4s-kvi8-ctx4096"), 300),
}


def run(name: str):
    cfg, P = RUNS[name]
    t0 = time.time()
    dec = oracle.Decoder.from_synth(cfg)
    pr = synth.prompt(cfg, P)
    print(f"{name}: weights in {time.time() - t0:.0f} s; {P} prompt positions", flush=True)
    toks, lgs = [], []
    nxt, lg = -1, None
    for p, t in enumerate(pr):
        nxt, lg = dec.step(int(t), p, want_logits=(p == P - 1))
        if p % 64 == 63:
            print(f"{name}: position {p + 1}/{P} at {time.time() - t0:.0f} s", flush=True)
    toks.append(nxt)
    lgs.append(lg)
    for i in range(N_EMIT - 1):
        nxt, lg = dec.step(toks[-1], P + i)
        toks.append(nxt)
        lgs.append(lg)
    gaps = []
    for l in lgs:
        s = np.sort(l)
        gaps.append(float(s[-1] - s[-2]))
    path = os.path.join(HERE, name + ".npz")
    np.savez_compressed(path, prompt=pr.astype(np.int32), tokens=np.array(toks, np.int32),
                        logits=np.stack(lgs).astype(np.float32),
                        top2_gap=np.array(gaps, np.float64))
    print(f"{name}: wrote {path} in {time.time() - t0:.0f} s; tokens {toks}; gaps {gaps}",
          flush=True)


def main():
    names = sys.argv[1:] or list(RUNS)
    for n in names:
        run(n)


if __name__ == "__main__":
    main()
