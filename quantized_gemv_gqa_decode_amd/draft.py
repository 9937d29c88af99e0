"""N-gram drafter for speculative greedy decode.

[k3_run.c] (the --spec option and spec_draft()): draft up to N tokens by
n-gram lookup in the sequence so far and verify them in one batched sweep; a
draft fires only where the earlier occurrences of the sequence's suffix agree
on what followed them.  Stated rules, as read here:

* match length 4, then 3: the suffix n-gram is the last n tokens, and its
  occurrences are the earlier positions where the same n tokens appear (an
  occurrence may overlap the suffix, but must leave at least one token after
  it inside the sequence);
* the draft copies what followed the most recent occurrence, token by token,
  and stops at the first position where ANY other occurrence's continuation
  disagrees ("every occurrence must propose the same next id ... stops at
  the first position where historical continuations diverge"), where the
  most recent continuation reaches the end of the sequence, or after
  MAX_DRAFT (8) tokens;
* a 4-gram whose occurrences disagree on the very first token yields no
  draft and the 3-gram is tried; no occurrence at either length means no
  draft (the step then runs as plain decode).

The page's function body inspects only the two most recent occurrences while
its comment states the rule for every occurrence; the stated rule is taken.
Its other comment speaks of n = 3, then 2; the match lengths attached to the
drafter's own rules (4, then 3) are taken.
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np

MAX_DRAFT = 8


def ngram_draft(history: Sequence[int], k: int = MAX_DRAFT, n_max: int = 4, n_min: int = 3) -> List[int]:
    """Up to min(k, MAX_DRAFT) proposed tokens to follow `history`."""
    cap = min(int(k), MAX_DRAFT)
    seq = np.asarray(history, dtype=np.int64)
    T = len(seq)
    if cap <= 0:
        return []
    for n in range(n_max, n_min - 1, -1):
        if T < n + 1:
            continue
        suffix = seq[T - n:]
        # windows starting at j = 0 .. T-n-1 (each leaves a token after it)
        win = np.lib.stride_tricks.sliding_window_view(seq[:T - 1], n)
        occ = np.nonzero(np.all(win == suffix, axis=1))[0]
        if len(occ) == 0:
            continue
        m1 = int(occ[-1])                       # the most recent occurrence
        others = occ[:-1]
        out: List[int] = []
        i = 0
        while len(out) < cap and m1 + n + i < T:
            cand = int(seq[m1 + n + i])
            if len(others) and np.any(seq[others + n + i] != cand):
                break
            out.append(cand)
            i += 1
        if out:
            return out
    return []
