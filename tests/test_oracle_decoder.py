"""Pins for the oracle's whole decode step.

* Incremental (cached, one position per call, liboracle) equals full
  recompute (oracle.brute, torch fp64 library routines, no cache) -- the
  analogue of the K3 engine's GATE 3, k3_run.c header "DECODE STRATEGY".
* The same holds for every weight format (fp32, bf16, fp8 E4M3 + row scale,
  MXFP4) and KV format (fp32, bf16, int8), for G = 1 and for n_kv = n_qh.
* The greedy token stream of the tiny fp32 workload is stored under
  tests/golden/ (written by tests/golden/make_golden.py, which calls only the
  oracle) and must stay identical.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_dense_fp32_greedy.json")


def _incremental_vs_full(cfg, n_decode=None):
    dec = oracle.Decoder.from_synth(cfg)
    pr = synth.prompt(cfg)
    toks, lg = dec.generate(pr, cfg.n_decode if n_decode is None else n_decode)
    seq = list(pr) + toks[:-1]
    full = brute.forward_full(cfg, brute.weights_from_decoder(dec), seq).numpy()
    ref = full[len(pr) - 1:]
    return toks, np.stack(lg), ref


@pytest.mark.parametrize("wdt,kvdt", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "i8"),
                                      ("fp8", "i8"), ("mxfp4", "i8"), ("mxfp4", "bf16"),
                                      ("q4s", "i8")])
def test_incremental_equals_full_recompute(wdt, kvdt):
    cfg = synth.TINY.replace(wdt=wdt, kvdt=kvdt)
    toks, lg, ref = _incremental_vs_full(cfg)
    assert np.abs(lg - ref).max() <= 1e-12
    assert list(ref.argmax(axis=1)) == toks


@pytest.mark.parametrize("change", [dict(groups=1), dict(n_kv=4), dict(n_kv=1),
                                    dict(head_dim=32, n_qh=2, n_kv=1)])
def test_incremental_equals_full_shape_variants(change):
    cfg = synth.TINY.replace(**change)
    toks, lg, ref = _incremental_vs_full(cfg, n_decode=6)
    assert np.abs(lg - ref).max() <= 1e-12
    assert list(ref.argmax(axis=1)) == toks


def test_teacher_forcing_reproduces_free_run():
    cfg = synth.TINY
    dec = oracle.Decoder.from_synth(cfg)
    pr = synth.prompt(cfg)
    toks, lg = dec.generate(pr, 8)
    dec2 = oracle.Decoder.from_synth(cfg)
    toks2, lg2 = dec2.generate(pr, 8, teacher=toks)
    assert toks2 == toks
    assert all(np.array_equal(a, b) for a, b in zip(lg, lg2))


def test_budget_is_clamped_to_capacity():
    cfg = synth.TINY.replace(cap=20)
    dec = oracle.Decoder.from_synth(cfg)
    toks, _ = dec.generate(synth.prompt(cfg), 100)
    assert len(toks) == 20 - cfg.prompt_len
    with pytest.raises(ValueError):
        dec.step(0, 20)
    with pytest.raises(ValueError):
        dec.step(cfg.vocab, 0)


def test_tiny_greedy_golden_stream():
    with open(GOLDEN) as f:
        g = json.load(f)
    cfg = synth.TINY
    assert g["config"] == cfg.name
    dec = oracle.Decoder.from_synth(cfg)
    pr = synth.prompt(cfg)
    assert list(map(int, pr)) == g["prompt"]
    toks, lg = dec.generate(pr, cfg.n_decode)
    assert toks == g["tokens"]
    top = [float(np.max(l)) for l in lg]
    assert np.allclose(top, g["top_logit"], rtol=0, atol=1e-12)
