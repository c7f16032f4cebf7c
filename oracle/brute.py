"""Pure-Python brute force of the Sol-Attn forward for tiny grids.

TEST INFRASTRUCTURE ONLY: a second, loop-by-loop statement of the same
definition as oracle.py (page "Sol-Attn: Accelerating Video Generation
Inference via On-the-Fly Attention Sparsification", §2 "Block-Sparse
Attention" for the mean-pooled proxy, §3 "Dynamic threshold routing" with the
row-max threshold form, §3 "Approximate correction" for the skipped-block
term). It uses only Python floats and lists, builds every term one at a time,
and is meant for N <= a few hundred and d <= 16.
"""
from __future__ import annotations

import math
from typing import List, Sequence


def _blocks(N: int, bsz: int) -> List[range]:
    return [range(s, min(s + bsz, N)) for s in range(0, N, bsz)]


def _mean(rows: Sequence[Sequence[float]], idx: range) -> List[float]:
    d = len(rows[0])
    acc = [0.0] * d
    for t in idx:
        for c in range(d):
            acc[c] += rows[t][c]
    return [a / len(idx) for a in acc]


def _dot(a: Sequence[float], b: Sequence[float]) -> float:
    total = 0.0
    for x, y in zip(a, b):
        total += x * y
    return total


def brute_head(q, k, v, Bq: int, Bk: int, tau: float):
    """Returns (out, s, keep) as nested lists for one head; q, k, v are [N][d]."""
    N, d = len(q), len(q[0])
    qblocks, kblocks = _blocks(N, Bq), _blocks(N, Bk)
    rt = math.sqrt(d)
    s = [[_dot(_mean(q, qi), _mean(k, kj)) / rt for kj in kblocks] for qi in qblocks]
    keep = []
    for row in s:
        top = max(row)
        keep.append([True if math.isinf(tau) else (x >= top - tau) for x in row])
    vbars = [_mean(v, kj) for kj in kblocks]
    out = [[0.0] * d for _ in range(N)]
    for i, qi in enumerate(qblocks):
        for r in qi:
            terms = []  # (logit, weight, value-vector)
            for j, kj in enumerate(kblocks):
                if keep[i][j]:
                    for t in kj:
                        terms.append((_dot(q[r], k[t]) / rt, 1.0, v[t]))
                else:
                    terms.append((s[i][j], float(len(kj)), vbars[j]))
            m = max(t[0] for t in terms)
            den = 0.0
            num = [0.0] * d
            for logit, w, val in terms:
                e = w * math.exp(logit - m)
                den += e
                for c in range(d):
                    num[c] += e * val[c]
            out[r] = [x / den for x in num]
    return out, s, keep
