"""Pins for the sampling oracle (oracle/sampling.py).

The generator is pinned to the published Philox4x32-10 known-answer vectors;
the filters to hand-computed cases and closed-form distributions.
"""
import json
import math
import os

import numpy as np

from oracle import sampling as S

HERE = os.path.dirname(os.path.abspath(__file__))


def test_philox_known_answer_vectors():
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    for v in kat["vectors"]:
        out = S.philox4x32_10([int(x, 16) for x in v["counter"]], [int(x, 16) for x in v["key"]])
        assert ["%08x" % w for w in out] == v["out"]


def test_uniform_range_and_mean():
    u = np.array([S.uniform(7, c) for c in range(20000)])
    assert u.min() >= 0.0 and u.max() < 1.0
    assert abs(u.mean() - 0.5) < 0.01
    assert np.all(u * 2 ** 24 == np.floor(u * 2 ** 24))              # 24-bit grid


def _freq(logits, n=20000, **kw):
    kw.setdefault("temperature", 1.0)
    kw.setdefault("top_k", len(logits))
    kw.setdefault("top_p", 1.0)
    kw.setdefault("min_p", 0.0)
    kw.setdefault("penalty", 1.0)
    kw.setdefault("prev", [])
    f = np.zeros(len(logits))
    for c in range(n):
        t, _ = S.sample(logits, seed=11, counter=c, **kw)
        f[t] += 1
    return f / n


LG = [0.0, math.log(2), math.log(3), math.log(4)]                   # p = (1, 2, 3, 4) / 10


def test_softmax_distribution():
    assert np.abs(_freq(LG) - np.array([0.1, 0.2, 0.3, 0.4])).max() < 0.015


def test_temperature_sharpens():
    want = np.array([1, 4, 9, 16]) / 30.0                          # T = 1/2 squares the ratios
    assert np.abs(_freq(LG, temperature=0.5) - want).max() < 0.015


def test_top_p_keeps_the_shortest_prefix():
    # sorted 0.4, 0.3, 0.2, 0.1: cumulative 0.4 < 0.6 <= 0.7 keeps two tokens
    assert np.abs(_freq(LG, top_p=0.6) - np.array([0, 0, 3 / 7, 4 / 7])).max() < 0.015


def test_min_p_drops_the_tail():
    # keep p >= 0.6 * 0.4 = 0.24: the 0.4 and 0.3 tokens
    assert np.abs(_freq(LG, min_p=0.6) - np.array([0, 0, 3 / 7, 4 / 7])).max() < 0.015


def test_top_k():
    assert np.abs(_freq(LG, top_k=2) - np.array([0, 0, 3 / 7, 4 / 7])).max() < 0.015


def test_repetition_penalty_hand_case():
    # [2, 1, -1, 0.5], ids 0 and 2 seen (0 twice), r = 2: [1, 1, -2, 0.5];
    # top-1 is the tie 0 / 1, the lower id wins
    lg = [2.0, 1.0, -1.0, 0.5]
    for c in range(5):
        t, _ = S.sample(lg, 1.0, 1, 1.0, 0.0, 2.0, [0, 2, 0], 3, c)
        assert t == 0
    # without the penalty, top-2 sampling never yields id 3
    f = _freq(lg, top_k=2)
    assert f[3] == 0 and f[2] == 0


def test_top_k_one_is_greedy():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal(1000)
    for c in range(10):
        t, _ = S.sample(lg, 0.7, 1, 0.9, 0.1, 1.3, [], 1, c)
        assert t == int(np.argmax(lg))


def test_top_k_zero_means_no_truncation():
    # k = 0 keeps every token: the draws equal those with k = vocab for any
    # filters, and the distribution is the plain softmax
    rng = np.random.default_rng(5)
    lg = rng.standard_normal(300) * 2
    for c in range(200):
        a = S.sample(lg, 0.7, 0, 0.9, 0.02, 1.3, [3, 7, 7, 250], 21, c)
        b = S.sample(lg, 0.7, 300, 0.9, 0.02, 1.3, [3, 7, 7, 250], 21, c)
        assert a == b
    assert np.abs(_freq(LG, top_k=0) - np.array([0.1, 0.2, 0.3, 0.4])).max() < 0.015


def test_penalty_applies_to_every_distinct_previous_id():
    # hundreds of previous ids (duplicates counted once): each penalised
    # logit is l / r (l > 0) or l * r, the rest untouched -- checked through
    # a draw with top-k = 1 (the argmax of the penalised logits)
    rng = np.random.default_rng(6)
    lg = rng.standard_normal(2000)
    prev = list(rng.integers(0, 2000, 700)) * 2
    pen = lg.copy()
    for t in set(prev):
        pen[t] = pen[t] / 1.5 if pen[t] > 0 else pen[t] * 1.5
    tok, _ = S.sample(lg, 1.0, 1, 1.0, 0.0, 1.5, prev, 1, 0)
    assert tok == int(np.argmax(pen))
