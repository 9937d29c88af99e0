"""Oracle of seeded token sampling from logits -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's CPU baseline import the
oracle; the HIP path never does.

The k2-burn page lists sampling as "temperature / top-k / top-p / min-p /
repetition-penalty" (its "Project layout", sampling.rs) and gives no more.
Reading taken here (the conventional order of those filters):
  1. repetition penalty r >= 1 on every distinct token id in `prev`:
     a logit l > 0 becomes l / r, otherwise l * r;
  2. temperature T > 0: z = l / T;
  3. top-k: keep the k largest z (ties: the lower token id first); k = 0
     means no truncation (every token stays a candidate);
  4. softmax over the kept tokens;
  5. top-p: in that order, keep the shortest prefix whose cumulative
     probability reaches top_p (at least one token);
  6. min-p: keep the tokens whose probability is >= min_p * the largest;
  7. draw u in [0, 1) and return the first kept token (same order) whose
     cumulative (unnormalised) probability exceeds u * the kept total.
u comes from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC 2011): key = (seed low 32 bits, seed high
32 bits), counter = (counter low, counter high, 0, 0); u = (first output
word >> 8) * 2^-24, exact in fp32 and fp64.
"""
from __future__ import annotations

import numpy as np

_M0, _M1 = 0xD2511F53, 0xCD9E8D57          # Philox4x32 round multipliers
_W0, _W1 = 0x9E3779B9, 0xBB67AE85          # key schedule (Weyl) increments
_MASK = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """The four 32-bit output words for a 4-word counter and a 2-word key."""
    c = [int(x) & _MASK for x in counter]
    k0, k1 = int(key[0]) & _MASK, int(key[1]) & _MASK
    for _ in range(10):
        p0 = _M0 * c[0]
        p1 = _M1 * c[2]
        hi0, lo0 = p0 >> 32, p0 & _MASK
        hi1, lo1 = p1 >> 32, p1 & _MASK
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
        k0 = (k0 + _W0) & _MASK
        k1 = (k1 + _W1) & _MASK
    return c


def uniform(seed: int, counter: int) -> float:
    w = philox4x32_10([counter & _MASK, (counter >> 32) & _MASK, 0, 0],
                      [seed & _MASK, (seed >> 32) & _MASK])
    return (w[0] >> 8) * 2.0 ** -24


def sample(logits, temperature: float, top_k: int, top_p: float, min_p: float,
           penalty: float, prev, seed: int, counter: int):
    """Returns (token, margin): margin is the smallest distance at which a
    decision of this draw is taken -- in z between the two tokens on either
    side of the top-k cut, in kept probability mass between top_p and the
    cumulative sums on either side of the top-p cut, between the min-p
    threshold and a probability it compares, between u * total and the
    cumulative sums on either side of the drawn token, and in z between the
    drawn token and its neighbours in the order -- where it is tiny, a
    computation in another precision may pick a neighbour."""
    l = np.asarray(logits, dtype=np.float64).copy()
    for t in sorted(set(int(x) for x in prev)):
        l[t] = l[t] / penalty if l[t] > 0 else l[t] * penalty
    z = l / temperature
    order = np.lexsort((np.arange(z.size), -z))                  # value desc, id asc
    margins = []
    if 0 < top_k < z.size:
        margins.append(abs(z[order[top_k - 1]] - z[order[top_k]]))
    if top_k > 0:
        order = order[:top_k]
    zk = z[order]
    p = np.exp(zk - zk[0])
    p /= p.sum()
    cum = np.cumsum(p)
    n = int(np.searchsorted(cum, top_p - 1e-15) + 1) if top_p < 1.0 else len(p)
    n = max(1, min(n, len(p)))
    if top_p < 1.0:
        margins += [abs(cum[j] - top_p) for j in (n - 2, n - 1) if 0 <= j < len(p)]
    keep = p[:n]
    ids = order[:n]
    zkeep = zk[:n]
    if min_p > 0.0:
        thr = min_p * keep[0]
        margins.append(float(np.abs(keep - thr).min()))
        if n < len(p):
            margins.append(abs(p[n] - thr))
        sel = keep >= thr
        keep, ids, zkeep = keep[sel], ids[sel], zkeep[sel]
    total = keep.sum()
    u = uniform(seed, counter)
    target = u * total
    acc = np.cumsum(keep)
    j = int(np.searchsorted(acc, target, side="right"))       # first cumulative > target
    j = min(j, len(keep) - 1)
    pick = int(ids[j])
    margins.append(abs(acc[j] - target))
    margins.append(abs((acc[j - 1] if j > 0 else 0.0) - target))
    for jj in (j - 1, j + 1):
        if 0 <= jj < len(zkeep):
            margins.append(abs(zkeep[jj] - zkeep[j]))
    return pick, (min(margins) if margins else 1.0)
