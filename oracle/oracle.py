"""fp64 CPU oracle of the Sol-Attn sparse attention forward.

TEST INFRASTRUCTURE ONLY. This module is the slow, obviously correct statement
of what the GPU path computes. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does. It
shares no code with the HIP kernels or their binding.

Sources (page "Sol-Attn: Accelerating Video Generation Inference via On-the-Fly
Attention Sparsification", paperlayer.ai summary of arXiv 2607.24027):

* §2 Preliminaries, "Attention and Online Softmax": attention is
  softmax(q k^T / sqrt(d)) v, evaluated without materialising the L x L map.
* §2 Preliminaries, "Block-Sparse Attention": the sequence is cut into query
  and key-value blocks; each block pair gets a proxy score from the MEAN of the
  query block and the MEAN of the key block.
* §3 Methodology, "Dynamic threshold routing": a query-dependent threshold on
  the proxy scores selects blocks. Its exact statistic is not printed; this
  implementation fixes it as the row maximum minus tau:
  keep(i, j) <=> s_ij >= max_j' s_ij' - tau  (tau in [0, +inf]; ties kept).
* §3 Methodology, "Approximate correction": selected blocks are computed
  exactly; every unselected block still contributes to the softmax numerator
  and denominator through its proxy score, using pooled keys and SUMMED values.
  Written out: a skipped block j adds exp(s_ij - m) * n_j * mean(v_j) to the
  numerator and exp(s_ij - m) * n_j to the denominator, n_j its token count.
* §3 Methodology, "Unified execution": one online-softmax state holds both the
  exact and the corrected terms, so the result is a single softmax over the
  union of exact token logits and block proxy logits.
* App. B, "Approximation error": keys are dense and non-causal within a block,
  so a block's mean is over all of its valid tokens (no masks).

Readings where the pages are silent (each is listed with its reason in the
project's design notes):
  - the proxy scale is 1/sqrt(d), the same as the exact logits;
  - the proxy is one value per (query block, key block) and serves every row of
    the query block;
  - a ragged last block pools only its valid tokens, n_j = its valid count;
  - pooling is the arithmetic mean for q, k and v.

Every function below computes in float64 on the values it is given.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, Optional

import numpy as np


def block_bounds(N: int, bsz: int) -> np.ndarray:
    """[nb, 2] half-open token ranges of consecutive blocks of size bsz; the
    last block holds the remainder (§2 "Block-Sparse Attention")."""
    nb = -(-N // bsz)
    starts = np.arange(nb, dtype=np.int64) * bsz
    stops = np.minimum(starts + bsz, N)
    return np.stack([starts, stops], axis=1)


def block_means(x: np.ndarray, bsz: int):
    """Mean of each block's rows over its valid tokens, and the token counts.

    §2 "Block-Sparse Attention" (mean-pooled blocks); §3 "Approximate
    correction" (pooled keys, and summed values = count * mean).
    """
    x = np.asarray(x, dtype=np.float64)
    bounds = block_bounds(x.shape[0], bsz)
    counts = (bounds[:, 1] - bounds[:, 0]).astype(np.float64)
    means = np.stack([x[a:b].sum(axis=0) / (b - a) for a, b in bounds])
    return means, counts


def proxy_scores(qbar: np.ndarray, kbar: np.ndarray, d: int) -> np.ndarray:
    """s_ij = qbar_i . kbar_j / sqrt(d)  (§2 "Block-Sparse Attention")."""
    return (np.asarray(qbar, np.float64) @ np.asarray(kbar, np.float64).T) / math.sqrt(d)


def route(s: np.ndarray, tau: float):
    """Row maxima M_i and the keep mask s_ij >= M_i - tau (§3 "Dynamic
    threshold routing", row-max form). tau = +inf keeps every block."""
    if not (tau >= 0.0):  # also rejects NaN
        raise ValueError("tau must be >= 0")
    M = s.max(axis=1)
    if math.isinf(tau):
        keep = np.ones_like(s, dtype=bool)
    else:
        keep = s >= (M - tau)[:, None]
    return M, keep


def gauss_threshold(qbar: np.ndarray, kbar: np.ndarray, d: int, beta: float) -> np.ndarray:
    """Query-dependent threshold theta_i = mu_i + beta * sigma_i from pooled-key
    moments (§3 "Dynamic threshold routing": the mean and variance of a proxy
    row come from first and second moments of the pooled keys, O(d^2) state;
    App. B "Threshold variance derivation").

    The statistics are over the key blocks j of a row, each block one sample:
      mu_i      = qbar_i . m_K / sqrt(d),           m_K = mean_j kbar_j
      sigma_i^2 = qbar_i^T C_K qbar_i / d,          C_K = mean_j (kbar_j - m_K)(kbar_j - m_K)^T
    (population moments). Nothing of size Nq x Nk is formed.
    """
    qbar = np.asarray(qbar, np.float64)
    kbar = np.asarray(kbar, np.float64)
    m_k = kbar.mean(axis=0)
    c = kbar - m_k
    C_k = (c.T @ c) / kbar.shape[0]
    mu = (qbar @ m_k) / math.sqrt(d)
    var = np.einsum("id,de,ie->i", qbar, C_k, qbar) / d
    return mu + beta * np.sqrt(np.maximum(var, 0.0))


def gauss_threshold_diag(qbar: np.ndarray, kbar: np.ndarray, d: int, beta: float) -> np.ndarray:
    """The diagonal estimator of the same threshold (App. B "Diagonal threshold
    estimator"): C_K replaced by its diagonal v_K = per-dimension variance of
    the pooled keys, so sigma_i^2 ~= sum_c qbar_ic^2 v_Kc / d, O(d) per block."""
    qbar = np.asarray(qbar, np.float64)
    kbar = np.asarray(kbar, np.float64)
    m_k = kbar.mean(axis=0)
    v_k = ((kbar - m_k) ** 2).mean(axis=0)
    mu = (qbar @ m_k) / math.sqrt(d)
    var = (qbar ** 2) @ v_k / d
    return mu + beta * np.sqrt(var)


def attend_head(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    Bq: int,
    Bk: int,
    tau: float,
    keep_override: Optional[np.ndarray] = None,
    query_blocks: Optional[Iterable[int]] = None,
    correction: bool = True,
    rule: str = "rowmax",
    beta: float = 0.0,
    sinks: Optional[tuple] = None,
    row_correction: bool = False,
) -> Dict[str, np.ndarray]:
    """Sparse-plus-corrected attention of one head; q, k, v are [N, d].

    For query block i with rows r:
      exact terms     : every token t of every kept block j, logit q_r.k_t/sqrt(d),
                        weight 1, value v_t;
      correction terms: every skipped block j, logit s_ij, weight n_j, value vbar_j;
      out_r = sum(weight*exp(logit-m)*value) / sum(weight*exp(logit-m)), m = max logit.

    ``keep_override`` ([Nq, Nk] bool) replaces the routing decision (used to
    condition on another implementation's choices at near-ties).
    ``query_blocks`` restricts the work to those query blocks; output rows of
    other blocks are NaN and their s/M/keep rows are NaN/False.
    ``correction=False`` drops the skipped blocks instead (the keep-or-drop
    "exact-only" baseline of §4 "Ablations", same selected blocks).
    ``rule`` picks the threshold: "rowmax" (keep s_ij >= max_j s_ij - tau),
    "gauss" (keep s_ij >= gauss_threshold, beta the standardized cutoff;
    tau is ignored) or "gauss_diag" (the diagonal estimator of it).
    ``sinks`` = (first, count): key blocks first .. first+count-1 are always
    kept in the exact branch (App. A: text key-value tokens retained as sinks).
    ``row_correction=True`` gives every row its own correction logit for a
    skipped block, q_r . kbar_j / sqrt(d) (one token-to-block score per row
    and key block, §3 "Unified execution"; App. B analyses one query row),
    instead of the block's s_ij; weight n_j and value vbar_j are unchanged.
    Routing stays block-level.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N, d = q.shape
    qb = block_bounds(N, Bq)
    kb = block_bounds(N, Bk)
    Nq, Nk = len(qb), len(kb)
    kbar, kcnt = block_means(k, Bk)
    vbar, _ = block_means(v, Bk)

    rows = np.arange(Nq) if query_blocks is None else np.array(sorted(set(query_blocks)), dtype=np.int64)
    qbar = np.stack([q[qb[i, 0]:qb[i, 1]].mean(axis=0) for i in rows]) if len(rows) else np.zeros((0, d))

    s = np.full((Nq, Nk), np.nan)
    M = np.full(Nq, np.nan)
    keep = np.zeros((Nq, Nk), dtype=bool)
    s_sel = proxy_scores(qbar, kbar, d)
    if rule == "rowmax":
        M_sel, keep_sel = route(s_sel, tau)
    elif rule in ("gauss", "gauss_diag"):
        if not math.isfinite(beta):
            raise ValueError("beta must be finite")
        theta = (gauss_threshold if rule == "gauss" else gauss_threshold_diag)(qbar, kbar, d, beta)
        M_sel = s_sel.max(axis=1) if s_sel.size else np.zeros(len(rows))
        keep_sel = s_sel >= theta[:, None]
    else:
        raise ValueError(f"unknown rule {rule!r}")
    if sinks is not None and sinks[1] > 0:
        first, count = sinks
        if first < 0 or first + count > Nk:
            raise ValueError("sink blocks out of range")
        keep_sel[:, first:first + count] = True
    s[rows], M[rows], keep[rows] = s_sel, M_sel, keep_sel
    if keep_override is not None:
        keep[rows] = np.asarray(keep_override, dtype=bool)[rows]

    out = np.full((N, d), np.nan)
    scale = 1.0 / math.sqrt(d)
    for i in rows:
        r0, r1 = qb[i]
        kept = np.flatnonzero(keep[i])
        skipped = np.flatnonzero(~keep[i]) if correction else np.zeros(0, dtype=np.int64)
        tok = (np.concatenate([np.arange(kb[j, 0], kb[j, 1]) for j in kept])
               if len(kept) else np.zeros(0, dtype=np.int64))
        x = (q[r0:r1] @ k[tok].T) * scale                     # exact logits [n_i, T]
        if row_correction:
            sc = (q[r0:r1] @ kbar[skipped].T) * scale             # token-to-block logits
        else:
            sc = np.broadcast_to(s[i, skipped], (r1 - r0, len(skipped)))  # proxy logits
        m = np.full(r1 - r0, -np.inf)
        if x.shape[1]:
            m = np.maximum(m, x.max(axis=1))
        if sc.shape[1]:
            m = np.maximum(m, sc.max(axis=1))
        e = np.exp(x - m[:, None])                            # weight 1 per token
        c = kcnt[skipped][None, :] * np.exp(sc - m[:, None])  # weight n_j per block
        den = e.sum(axis=1) + c.sum(axis=1)
        num = e @ v[tok] + c @ vbar[skipped]
        out[r0:r1] = num / den[:, None]

    kept_counts = keep.sum(axis=1)
    return {"out": out, "s": s, "M": M, "keep": keep, "kept_counts": kept_counts,
            "rows": rows}


def attend(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    Bq: int,
    Bk: int,
    tau: float,
    keep_override: Optional[np.ndarray] = None,
    query_blocks: Optional[Iterable[int]] = None,
) -> Dict[str, np.ndarray]:
    """attend_head over every head of [B, H, N, d] inputs.

    keep_override, if given, is [B, H, Nq, Nk]. Returns out [B, H, N, d] and
    s, M, keep stacked per head.
    """
    B, H, N, d = q.shape
    outs, ss, Ms, keeps = [], [], [], []
    for b in range(B):
        for h in range(H):
            r = attend_head(
                q[b, h], k[b, h], v[b, h], Bq, Bk, tau,
                None if keep_override is None else keep_override[b, h],
                query_blocks,
            )
            outs.append(r["out"]); ss.append(r["s"]); Ms.append(r["M"]); keeps.append(r["keep"])
    Nq, Nk = ss[0].shape
    return {
        "out": np.stack(outs).reshape(B, H, N, d),
        "s": np.stack(ss).reshape(B, H, Nq, Nk),
        "M": np.stack(Ms).reshape(B, H, Nq),
        "keep": np.stack(keeps).reshape(B, H, Nq, Nk),
    }


def route_head(q: np.ndarray, k: np.ndarray, Bq: int, Bk: int, tau: float):
    """Proxy scores, row maxima and keep mask of one head, without outputs."""
    d = q.shape[1]
    qbar, _ = block_means(q, Bq)
    kbar, _ = block_means(k, Bk)
    s = proxy_scores(qbar, kbar, d)
    M, keep = route(s, tau)
    return s, M, keep


def topk_mask(s: np.ndarray, k: int) -> np.ndarray:
    """Keep the k highest proxy scores of each row, a fixed budget (§2
    "Block-Sparse Attention": top-k routing). Equal scores are taken in order
    of increasing block index. k is clipped to [0, Nk]."""
    s = np.asarray(s, np.float64)
    nk = s.shape[1]
    k = max(0, min(int(k), nk))
    keep = np.zeros(s.shape, dtype=bool)
    for i in range(s.shape[0]):
        order = sorted(range(nk), key=lambda j: (-s[i, j], j))
        keep[i, order[:k]] = True
    return keep


def topp_mask(s: np.ndarray, p: float) -> np.ndarray:
    """Keep, per row, the fewest highest-scoring blocks whose share of the
    row's softmax mass over the proxy scores reaches p (§2 "Block-Sparse
    Attention": top-p routing, a dynamic budget). Scores are taken from the
    highest down, equal scores in order of increasing block index; the block
    at which the running share first reaches p is kept. p <= 0 keeps the top
    block only; p >= 1 keeps every block."""
    s = np.asarray(s, np.float64)
    nk = s.shape[1]
    keep = np.zeros(s.shape, dtype=bool)
    for i in range(s.shape[0]):
        order = sorted(range(nk), key=lambda j: (-s[i, j], j))
        w = np.exp(s[i, order] - s[i, order[0]])
        share = np.cumsum(w) / w.sum()
        reach = np.flatnonzero(share >= p)
        last = int(reach[0]) if len(reach) else nk - 1
        keep[i, order[:last + 1]] = True
    return keep
