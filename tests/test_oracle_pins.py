"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each test names the passage of the page "Sol-Attn: Accelerating Video
Generation Inference via On-the-Fly Attention Sparsification" (paperlayer.ai
summary) or the mathematical fact it relies on. Together they are chosen so
that a dropped term, a wrong sign, a wrong block index, a transposed operand,
a sum taken for a mean or a missing token count fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (attend, attend_head, block_means, gauss_threshold, gauss_threshold_diag, route, topk_mask,
                    topp_mask)
from oracle.brute import brute_head

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def sdpa64(q, k, v):
    """Dense softmax attention from torch's library routine, fp64 on the CPU."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))[0, 0].numpy()


def rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


# ---------------------------------------------------------------------------
# Hand-derived worked examples (closed forms in e)
# ---------------------------------------------------------------------------

def _closed(expr):
    return eval(expr, {"__builtins__": {}}, {"e": math.e})  # noqa: S307 - fixed fixture strings


@pytest.mark.parametrize("ex", json.load(open(GOLDEN))["examples"], ids=lambda ex: ex["name"])
def test_worked_examples(ex):
    N, d = ex["N"], ex["d"]
    tau = math.inf if ex["tau"] == "inf" else float(ex["tau"])
    q = np.array(ex["q"], dtype=np.float64).reshape(N, d)
    k = np.array(ex["k"], dtype=np.float64).reshape(N, d)
    v = np.array(ex["v"], dtype=np.float64).reshape(N, d)
    r = attend_head(q, k, v, ex["Bq"], ex["Bk"], tau)
    assert r["keep"].tolist() == ex["keep"]
    np.testing.assert_allclose(r["s"].ravel(), [_closed(x) for x in ex["s"]], rtol=0, atol=1e-14)
    np.testing.assert_allclose(r["out"].ravel(), [_closed(x) for x in ex["out"]], rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------------------
# tau = +inf is dense softmax attention (§2 "Attention and Online Softmax";
# §3 "Approximate correction": selected blocks are computed exactly)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,d,Bq,Bk", [(1000, 16, 64, 64), (200, 8, 32, 48), (130, 4, 7, 13), (64, 32, 64, 64)])
def test_dense_limit_equals_sdpa(N, d, Bq, Bk):
    rng = np.random.default_rng(N * 7 + d)
    q, k, v = rand(rng, N, d, scale=2.0), rand(rng, N, d, scale=2.0), rand(rng, N, d)
    r = attend_head(q, k, v, Bq, Bk, math.inf)
    assert r["keep"].all()
    np.testing.assert_allclose(r["out"], sdpa64(q, k, v), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Brute force on tiny grids: proxies, keep mask and outputs term by term
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,d,Bq,Bk", [(5, 3, 2, 2), (16, 4, 4, 4), (37, 3, 8, 5), (40, 8, 16, 8), (23, 2, 23, 4)])
@pytest.mark.parametrize("tau", [0.0, 0.3, 1.0, 3.0, math.inf])
def test_brute_force_tiny(N, d, Bq, Bk, tau):
    rng = np.random.default_rng(1000 * N + 10 * d + Bq)
    q, k, v = rand(rng, N, d, scale=1.5), rand(rng, N, d, scale=1.5), rand(rng, N, d)
    r = attend_head(q, k, v, Bq, Bk, tau)
    out_b, s_b, keep_b = brute_head(q.tolist(), k.tolist(), v.tolist(), Bq, Bk, tau)
    np.testing.assert_allclose(r["s"], np.array(s_b), rtol=0, atol=1e-12)
    assert (r["keep"] == np.array(keep_b)).all()
    np.testing.assert_allclose(r["out"], np.array(out_b), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Constant blocks: the zeroth-order correction is exact (§3 "Approximate
# correction"; App. B "Approximation error": the error vanishes when the
# centred score deviations inside a block are zero)
# ---------------------------------------------------------------------------

def _block_constant(rng, N, d, bsz, scale):
    x = np.empty((N, d))
    for s in range(0, N, bsz):
        x[s:s + bsz] = rng.standard_normal(d) * scale
    return x


@pytest.mark.parametrize("N,Bq,Bk", [(1000, 64, 64), (1000, 48, 64), (777, 64, 100), (129, 64, 64)])
@pytest.mark.parametrize("v_kind", ["arbitrary", "block_constant"])
def test_tau0_constant_blocks_equals_dense(N, Bq, Bk, v_kind):
    d = 16
    rng = np.random.default_rng(N + Bq + Bk)
    q = _block_constant(rng, N, d, Bq, 1.5)
    k = _block_constant(rng, N, d, Bk, 1.5)
    v = rand(rng, N, d) if v_kind == "arbitrary" else _block_constant(rng, N, d, Bk, 1.0)
    r = attend_head(q, k, v, Bq, Bk, 0.0)
    assert (~r["keep"]).sum() > 0  # the correction path is exercised
    np.testing.assert_allclose(r["out"], sdpa64(q, k, v), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Routing invariants (§3 "Dynamic threshold routing", row-max form)
# ---------------------------------------------------------------------------

def test_routing_monotone_in_tau_and_argmax_kept():
    rng = np.random.default_rng(7)
    N, d = 640, 16
    q, k = rand(rng, N, d, scale=2.0), rand(rng, N, d, scale=2.0)
    qbar, _ = block_means(q, 64)
    kbar, _ = block_means(k, 64)
    s = qbar @ kbar.T / math.sqrt(d)
    prev = None
    for tau in [0.0, 0.1, 0.5, 1.0, 2.0, 4.0, math.inf]:
        M, keep = route(s, tau)
        assert keep[np.arange(len(M)), s.argmax(axis=1)].all()
        assert keep.sum(axis=1).min() >= 1
        if prev is not None:
            assert (prev <= keep).all()
        prev = keep
    # with distinct scores, tau = 0 keeps exactly the argmax
    M, keep = route(s, 0.0)
    assert (keep.sum(axis=1) == 1).all()


@pytest.mark.parametrize("N,d,Bq,Bk", [(37, 3, 8, 5), (40, 4, 16, 8), (23, 2, 4, 23), (61, 5, 7, 12), (64, 3, 64, 16)])
@pytest.mark.parametrize("tau", [0.0, 0.4, 2.0, math.inf])
def test_route_head_matches_brute_force_and_attend_head(N, d, Bq, Bk, tau):
    """route_head (the routing-only entry of the oracle) against the
    pure-Python brute force (§2 "Block-Sparse Attention": means of the query
    and key blocks, one score per block pair) and against attend_head's own
    routing. Unequal block sizes on both sides, with ragged last blocks, make
    a swapped Bq/Bk fail; non-centred inputs (a common offset) make a sum
    taken for a mean change every score."""
    from oracle import route_head

    rng = np.random.default_rng(31 * N + 7 * d + Bq + Bk)
    q = rand(rng, N, d, scale=1.5) + 0.7
    k = rand(rng, N, d, scale=1.5) - 0.4
    v = rand(rng, N, d)
    s, M, keep = route_head(q, k, Bq, Bk, tau)
    _, s_b, keep_b = brute_head(q.tolist(), k.tolist(), v.tolist(), Bq, Bk, tau)
    s_b = np.array(s_b)
    assert s.shape == (-(-N // Bq), -(-N // Bk))
    np.testing.assert_allclose(s, s_b, rtol=0, atol=1e-12)
    np.testing.assert_allclose(M, s_b.max(axis=1), rtol=0, atol=1e-12)
    assert (keep == np.array(keep_b)).all()
    r = attend_head(q, k, v, Bq, Bk, tau)
    np.testing.assert_allclose(s, r["s"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(M, r["M"], rtol=0, atol=1e-12)
    assert (keep == r["keep"]).all()


def test_route_rejects_negative_or_nan_tau():
    s = np.zeros((2, 2))
    for bad in (-1e-9, -1.0, float("nan")):
        with pytest.raises(ValueError):
            route(s, bad)


def test_single_kv_block_is_dense():
    rng = np.random.default_rng(11)
    N, d = 50, 8
    q, k, v = rand(rng, N, d, scale=3.0), rand(rng, N, d, scale=3.0), rand(rng, N, d)
    r = attend_head(q, k, v, 16, 64, 0.0)
    assert r["keep"].all()
    np.testing.assert_allclose(r["out"], sdpa64(q, k, v), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Output algebra: the result is a convex combination of token values and
# block mean values
# ---------------------------------------------------------------------------

def test_value_shift_invariance_and_convex_hull():
    rng = np.random.default_rng(3)
    N, d = 300, 8
    q, k, v = rand(rng, N, d, scale=2.0), rand(rng, N, d, scale=2.0), rand(rng, N, d)
    c = rng.standard_normal(d)
    for tau in (0.0, 1.0, 3.0):
        a = attend_head(q, k, v, 32, 32, tau)["out"]
        b = attend_head(q, k, v + c, 32, 32, tau)["out"]
        np.testing.assert_allclose(b, a + c, rtol=0, atol=1e-12)
        assert (a <= v.max(axis=0) + 1e-12).all() and (a >= v.min(axis=0) - 1e-12).all()


def test_kv_block_permutation_invariance():
    rng = np.random.default_rng(5)
    Bk, nb, d = 16, 9, 8
    N = Bk * nb
    q, k, v = rand(rng, N, d, scale=2.0), rand(rng, N, d, scale=2.0), rand(rng, N, d)
    perm = rng.permutation(nb)
    idx = np.concatenate([np.arange(j * Bk, (j + 1) * Bk) for j in perm])
    for tau in (0.0, 0.7, 2.0):
        a = attend_head(q, k, v, 24, Bk, tau)
        b = attend_head(q, k[idx], v[idx], 24, Bk, tau)
        np.testing.assert_allclose(b["out"], a["out"], rtol=0, atol=1e-12)
        assert (b["keep"] == a["keep"][:, perm]).all()


def test_token_permutation_inside_block_invariance():
    """Inside a block only the block's mean and its tokens as a set matter."""
    rng = np.random.default_rng(9)
    N, d, Bk = 160, 8, 32
    q, k, v = rand(rng, N, d, scale=2.0), rand(rng, N, d, scale=2.0), rand(rng, N, d)
    idx = np.concatenate([s + rng.permutation(min(Bk, N - s)) for s in range(0, N, Bk)])
    a = attend_head(q, k, v, 32, Bk, 1.0)["out"]
    b = attend_head(q, k[idx], v[idx], 32, Bk, 1.0)["out"]
    np.testing.assert_allclose(b, a, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# App. B "Approximation error": for a skipped block, the denominator error is
# second order in the centred score spread; the numerator error is first order
# with a coefficient set by the alignment of the deviations with the values.
# ---------------------------------------------------------------------------

def _scaling_case(eps, aligned):
    rng = np.random.default_rng(21)
    d, Bk = 8, 32
    qv = rng.standard_normal(d)
    q = np.tile(qv, (Bk, 1))                            # one query block, constant rows
    k0 = np.tile(qv * 0.8, (Bk, 1))                     # block 0: strongly aligned, kept
    kbar1 = -0.1 * qv + 0.05 * rng.standard_normal(d)   # block 1: far below, skipped
    delta = rng.standard_normal((Bk, d))
    delta -= delta.mean(axis=0)                         # zero-mean deviations
    k1 = kbar1 + eps * delta
    k = np.concatenate([k0, k1])
    v0 = rng.standard_normal((Bk, d))
    if aligned:
        a = delta @ qv / math.sqrt(d)                   # centred score deviations
        v1 = 0.3 + np.outer(a, np.ones(d))
    else:
        v1 = np.full((Bk, d), 0.3)
    v = np.concatenate([v0, v1])
    qq = np.concatenate([q, q])
    r = attend_head(qq, k, v, Bk, Bk, 1.0)
    assert r["keep"].tolist() == [[True, False], [True, False]]
    return np.abs(r["out"] - sdpa64(qq, k, v)).max()


@pytest.mark.parametrize("aligned,ratio", [(False, 4.0), (True, 2.0)])
def test_error_order_in_score_spread(aligned, ratio):
    e1 = _scaling_case(2e-2, aligned)
    e2 = _scaling_case(1e-2, aligned)
    assert e1 > 0 and e2 > 0
    assert abs(e1 / e2 - ratio) < 0.15 * ratio, (e1, e2, e1 / e2)


# ---------------------------------------------------------------------------
# Oracle plumbing: sub-selection and override agree with the full computation
# ---------------------------------------------------------------------------

def test_query_block_subset_and_override_consistent():
    rng = np.random.default_rng(13)
    N, d = 700, 16
    q, k, v = rand(rng, N, d, scale=2.0), rand(rng, N, d, scale=2.0), rand(rng, N, d)
    full = attend_head(q, k, v, 64, 64, 2.0)
    sub = attend_head(q, k, v, 64, 64, 2.0, query_blocks=[0, 5, 10])
    for i in (0, 5, 10):
        r0, r1 = i * 64, min(N, i * 64 + 64)
        np.testing.assert_array_equal(sub["out"][r0:r1], full["out"][r0:r1])
        np.testing.assert_array_equal(sub["keep"][i], full["keep"][i])
    assert np.isnan(sub["out"][64:128]).all()
    over = attend_head(q, k, v, 64, 64, 0.0, keep_override=full["keep"])
    np.testing.assert_allclose(over["out"], full["out"], rtol=0, atol=1e-13)


def test_batched_attend_matches_per_head():
    rng = np.random.default_rng(17)
    B, H, N, d = 2, 3, 150, 8
    q, k, v = (rand(rng, B, H, N, d, scale=2.0) for _ in range(3))
    r = attend(q, k, v, 32, 32, 1.5)
    for b in range(B):
        for h in range(H):
            one = attend_head(q[b, h], k[b, h], v[b, h], 32, 32, 1.5)
            np.testing.assert_array_equal(r["out"][b, h], one["out"])
            np.testing.assert_array_equal(r["keep"][b, h], one["keep"])


# ---------------------------------------------------------------------------
# Exact-only (keep-or-drop) baseline of §4 "Ablations": softmax attention
# restricted to the tokens of the kept blocks, i.e. a masked library SDPA.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,Bq,Bk,tau", [(300, 32, 32, 0.2), (250, 64, 48, 0.1), (130, 16, 64, 0.0)])
def test_exact_only_equals_masked_sdpa(N, Bq, Bk, tau):
    rng = np.random.default_rng(N + Bk)
    d = 8
    q, k, v = rand(rng, N, d, scale=2.0), rand(rng, N, d, scale=2.0), rand(rng, N, d)
    r = attend_head(q, k, v, Bq, Bk, tau, correction=False)
    mask = np.zeros((N, N), dtype=bool)
    for i in range(r["keep"].shape[0]):
        for j in np.flatnonzero(r["keep"][i]):
            mask[i * Bq:(i + 1) * Bq, j * Bk:(j + 1) * Bk] = True
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=torch.from_numpy(mask))[0, 0]
    np.testing.assert_allclose(r["out"], ref.numpy(), rtol=0, atol=1e-12)
    assert (~r["keep"]).any()


# ---------------------------------------------------------------------------
# Gaussian-calibrated threshold (§3 "Dynamic threshold routing"; App. B
# "Threshold variance derivation", "Diagonal threshold estimator") and
# forced-keep sink blocks (App. A)
# ---------------------------------------------------------------------------

GAUSS_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gauss_sink_examples.json")


@pytest.mark.parametrize("case", json.load(open(GAUSS_GOLDEN))["cases"], ids=lambda c: c["name"])
def test_gauss_and_sink_worked_examples(case):
    ex = json.load(open(GAUSS_GOLDEN))
    N, d = ex["N"], ex["d"]
    q, k, v = (np.array(ex[n], dtype=np.float64).reshape(N, d) for n in "qkv")
    sinks = tuple(case["sinks"]) if "sinks" in case else None
    r = attend_head(q, k, v, ex["Bq"], ex["Bk"], case.get("tau", 0.0), rule=case["rule"],
                    beta=case.get("beta", 0.0), sinks=sinks)
    assert r["keep"].tolist() == case["keep"]
    np.testing.assert_allclose(r["s"][0], [_closed(x) for x in ex["s"]], rtol=0, atol=1e-14)
    np.testing.assert_allclose(r["out"].ravel(), _closed(case["out"]), rtol=1e-13, atol=1e-14)
    if case["rule"] == "gauss":
        qbar, _ = block_means(q, ex["Bq"])
        kbar, _ = block_means(k, ex["Bk"])
        np.testing.assert_allclose(gauss_threshold(qbar, kbar, d, case["beta"]), _closed(case["theta"]),
                                   rtol=0, atol=1e-14)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_gauss_threshold_from_moments_equals_row_statistics(seed):
    """The moment form never builds the proxy row; its mean and population
    standard deviation must still be those of the row, which numpy computes
    here directly from the row."""
    rng = np.random.default_rng(seed)
    d, Nq, Nk = 16, 9, 37
    qbar = rand(rng, Nq, d) + 0.5
    kbar = rand(rng, Nk, d) @ rand(rng, d, d) * 0.3 + rand(rng, d)  # correlated, off-centre
    s = (qbar @ kbar.T) / math.sqrt(d)
    for beta in (-1.3, 0.0, 0.7, 2.5):
        np.testing.assert_allclose(gauss_threshold(qbar, kbar, d, beta), s.mean(axis=1) + beta * s.std(axis=1),
                                   rtol=1e-12, atol=1e-12)


def test_gauss_diagonal_estimator():
    """Exact when the pooled keys' covariance is diagonal (columns centred and
    mutually orthogonal), different otherwise."""
    d = 4
    H = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]], dtype=np.float64)
    kbar = np.vstack([H[:, 1:], -H[:, 1:]]) * np.array([1.0, 2.0, 0.5]) + np.array([0.3, -0.2, 0.1])
    kbar = np.hstack([kbar, np.zeros((8, 1))])  # d = 4: the last dimension never varies
    c = kbar - kbar.mean(axis=0)
    cov = c.T @ c / len(kbar)
    assert np.allclose(cov, np.diag(np.diag(cov)))
    qbar = np.random.default_rng(3).standard_normal((5, d))
    for beta in (-1.0, 0.5, 2.0):
        np.testing.assert_allclose(gauss_threshold_diag(qbar, kbar, d, beta), gauss_threshold(qbar, kbar, d, beta),
                                   rtol=1e-12, atol=1e-12)
    kc = kbar.copy()
    kc[:, 1] += kc[:, 0]  # correlate two dimensions
    assert not np.allclose(gauss_threshold_diag(qbar, kc, d, 1.0), gauss_threshold(qbar, kc, d, 1.0))


def test_gauss_routing_monotone_in_beta_and_dense_limit():
    rng = np.random.default_rng(11)
    N, d = 700, 8
    q, k, v = rand(rng, N, d), rand(rng, N, d), rand(rng, N, d)
    prev = None
    for beta in (3.0, 1.0, 0.0, -1.0):
        keep = attend_head(q, k, v, 64, 64, 0.0, rule="gauss", beta=beta)["keep"]
        if prev is not None:
            assert (prev <= keep).all()  # a lower cutoff keeps a superset
        prev = keep
    r = attend_head(q, k, v, 64, 64, 0.0, rule="gauss", beta=-1e6)
    assert r["keep"].all()
    np.testing.assert_allclose(r["out"], sdpa64(q, k, v), rtol=1e-12, atol=1e-12)
    with pytest.raises(ValueError):
        attend_head(q, k, v, 64, 64, 0.0, rule="gauss", beta=math.nan)


def test_sinks_are_always_kept_and_all_sinks_is_dense():
    rng = np.random.default_rng(12)
    N, d = 640, 8
    q, k, v = rand(rng, N, d), rand(rng, N, d), rand(rng, N, d)
    r = attend_head(q, k, v, 64, 64, 0.0, sinks=(2, 3))
    assert r["keep"][:, 2:5].all()
    base = attend_head(q, k, v, 64, 64, 0.0)["keep"]
    assert (r["keep"][:, :2] == base[:, :2]).all() and (r["keep"][:, 5:] == base[:, 5:]).all()
    rd = attend_head(q, k, v, 64, 64, 0.0, sinks=(0, 10))
    np.testing.assert_allclose(rd["out"], sdpa64(q, k, v), rtol=1e-12, atol=1e-12)
    with pytest.raises(ValueError):
        attend_head(q, k, v, 64, 64, 0.0, sinks=(8, 3))


def test_correction_beats_exact_only_on_a_smooth_layer():
    """§4 "Ablations": with the same selected blocks, the corrected output is
    closer to dense attention than the exact-only one. A statistical property
    of smooth activations; pinned on one seeded, video-like layer whose
    queries, keys and values share a positional component (values that are
    independent per token have block means near zero, and there the two
    outputs nearly coincide)."""
    from workloads.gen import pos_code

    grid, d = (4, 16, 16), 64
    N = grid[0] * grid[1] * grid[2]
    P = pos_code(grid, d).astype(np.float64)
    rng = np.random.default_rng(5)
    q = rand(rng, N, d) + 3 * P
    k = rand(rng, N, d) + 3 * P
    v = rand(rng, N, d) + 3 * P
    dense = sdpa64(q, k, v)
    for tau in (0.5, 1.0, 2.0):
        c = attend_head(q, k, v, 64, 64, tau)["out"]
        e = attend_head(q, k, v, 64, 64, tau, correction=False)["out"]
        err_c = np.linalg.norm(c - dense) / np.linalg.norm(dense)
        err_e = np.linalg.norm(e - dense) / np.linalg.norm(dense)
        assert err_c < err_e, (tau, err_c, err_e)


def test_correction_order_on_a_mild_layer():
    """§4 "Ablations" and App. B: on a layer built like video_dit_32k_mild
    (milder locality, half-scale per-token draws of q and k, smooth values),
    reduced to a 4x16x32 grid at d = 128, the skipped blocks hold a visible
    share of the attention mass, and the outputs order as the pages describe:
    token-to-block correction closer to dense attention than block-level
    correction, which is closer than exact-only attention on the same blocks."""
    from workloads.gen import pos_code

    grid, d = (4, 16, 32), 128
    N = grid[0] * grid[1] * grid[2]
    P = pos_code(grid, d).astype(np.float64)
    rng = np.random.default_rng(11)
    q = 0.5 * rng.standard_normal((N, d)) + 1.5 * P
    k = 0.5 * rng.standard_normal((N, d)) + 1.5 * P
    v = rng.standard_normal((N, d)) + 3 * P
    dense = sdpa64(q, k, v)

    def err(o):
        return np.linalg.norm(o - dense) / np.linalg.norm(dense)

    for tau in (1.0, 2.0):
        row = err(attend_head(q, k, v, 64, 64, tau, row_correction=True)["out"])
        blk = err(attend_head(q, k, v, 64, 64, tau)["out"])
        exact = err(attend_head(q, k, v, 64, 64, tau, correction=False)["out"])
        assert row < blk < exact, (tau, row, blk, exact)
        assert blk < 0.8 * exact, (tau, blk, exact)


# ---------------------------------------------------------------------------
# Top-k and top-p masks, the routing baselines of §2 "Block-Sparse Attention"
# ---------------------------------------------------------------------------

def test_topk_topp_worked_example():
    """s = [0, 1, 2, 3]: softmax shares e^j / (1 + e + e^2 + e^3), from the top
    0.6439, 0.2369, 0.0871, 0.0321 (cumulative 0.6439, 0.8808, 0.9679, 1)."""
    s = np.array([[0.0, 1.0, 2.0, 3.0], [3.0, 2.0, 1.0, 0.0]])
    assert topk_mask(s, 1).tolist() == [[False, False, False, True], [True, False, False, False]]
    assert topk_mask(s, 3).tolist() == [[False, True, True, True], [True, True, True, False]]
    assert topk_mask(s, 0).sum() == 0 and topk_mask(s, 9).all()
    e = math.e
    z = 1 + e + e * e + e ** 3
    top1, top2, top3 = e ** 3 / z, (e ** 3 + e * e) / z, (e ** 3 + e * e + e) / z
    assert topp_mask(s, top1 - 1e-9)[0].tolist() == [False, False, False, True]
    assert topp_mask(s, top1 + 1e-9)[0].tolist() == [False, False, True, True]
    assert topp_mask(s, top2 + 1e-9)[0].tolist() == [False, True, True, True]
    assert topp_mask(s, top3 + 1e-9)[0].tolist() == [True, True, True, True]
    assert topp_mask(s, 0.0).sum(axis=1).tolist() == [1, 1]
    assert topp_mask(s, 1.0).all()


def test_topk_ties_by_index_and_budget():
    s = np.array([[1.0, 2.0, 2.0, 2.0, 0.0]])
    assert topk_mask(s, 2).tolist() == [[False, True, True, False, False]]
    rng = np.random.default_rng(4)
    s = rng.standard_normal((7, 40))
    for k in (1, 5, 40):
        m = topk_mask(s, k)
        assert (m.sum(axis=1) == k).all()
        # every kept score is at least every dropped one
        for i in range(7):
            if k < 40:
                assert s[i, m[i]].min() >= s[i, ~m[i]].max()


def test_topp_is_the_smallest_top_set_reaching_p():
    rng = np.random.default_rng(6)
    s = rng.standard_normal((9, 50)) * 2
    for p in (0.3, 0.7, 0.95):
        m = topp_mask(s, p)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        share = (w * m).sum(axis=1) / w.sum(axis=1)
        assert (share >= p - 1e-12).all()
        for i in range(9):
            kept = np.flatnonzero(m[i])
            assert s[i, kept].min() >= s[i, ~m[i]].max() if (~m[i]).any() else True
            # dropping the smallest kept block falls below p
            smallest = kept[np.argmin(s[i, kept])]
            assert (w[i, kept].sum() - w[i, smallest]) / w[i].sum() < p


# ---------------------------------------------------------------------------
# Token-to-block (per-row) correction (§3 "Unified execution": one shared
# token-to-block score tile; App. B "Approximation error" for one query row)
# ---------------------------------------------------------------------------

def test_row_correction_worked_example():
    """d = 1, one query block of two rows q = (1, 3) (qbar = 2), key blocks
    k = (0, 0 | 1, 1), v = (1, 1 | 2, 4), tau = 0.5: s = (0, 2), block 1 kept.
    Row q=1: exact terms e^1 (v=2), e^1 (v=4); block 0 corrected with the
    row's own logit 1*0 = 0, weight 2, vbar = 1: (6e + 2)/(2e + 2).
    Row q=3: (6e^3 + 2)/(2e^3 + 2). Block-level correction uses s = 0 for both
    rows here too (kbar_0 = 0), so take a shifted block: k = (1, 1 | 3, 3),
    s = (2, 6), kbar = (1, 3): row logits for block 0 are 1 and 3."""
    q = np.array([[1.0], [3.0]])
    k = np.array([[1.0], [1.0], [3.0], [3.0]])
    v = np.array([[1.0], [1.0], [2.0], [4.0]])
    q4 = np.vstack([q, q])  # two query blocks, the same rows
    e = math.e
    r = attend_head(q4, k, v, 2, 2, 0.5, row_correction=True)
    assert r["keep"].tolist() == [[False, True], [False, True]]
    row1 = (6 * e ** 3 + 2 * e) / (2 * e ** 3 + 2 * e)     # exact e^3 (v 2, 4); corrected 2 e^1 * 1
    row3 = (6 * e ** 9 + 2 * e ** 3) / (2 * e ** 9 + 2 * e ** 3)
    np.testing.assert_allclose(r["out"][:2, 0], [row1, row3], rtol=1e-14)
    # block-level: both rows use s_00 = qbar * kbar_0 = 2
    b = attend_head(q4, k, v, 2, 2, 0.5)
    blk1 = (6 * e ** 3 + 2 * e ** 2) / (2 * e ** 3 + 2 * e ** 2)
    blk3 = (6 * e ** 9 + 2 * e ** 2) / (2 * e ** 9 + 2 * e ** 2)
    np.testing.assert_allclose(b["out"][:2, 0], [blk1, blk3], rtol=1e-14)


def test_row_correction_exact_for_constant_key_blocks():
    """Keys constant inside every block make each token's logit equal the
    row's token-to-block logit, so the per-row correction is exact for any
    queries and values (tau = 0 keeps almost nothing); the block-level one is
    not, because queries vary inside a block."""
    rng = np.random.default_rng(21)
    N, d, Bk = 640, 8, 64
    q, v = rand(rng, N, d), rand(rng, N, d)
    kb = rand(rng, N // Bk, d)
    k = np.repeat(kb, Bk, axis=0)
    dense = sdpa64(q, k, v)
    r = attend_head(q, k, v, 64, Bk, 0.0, row_correction=True)
    assert r["keep"].sum() < r["keep"].size  # blocks were skipped
    np.testing.assert_allclose(r["out"], dense, rtol=1e-11, atol=1e-12)
    b = attend_head(q, k, v, 64, Bk, 0.0)
    assert np.abs(b["out"] - dense).max() > 1e-3


def test_query_and_key_spread_error_orders():
    """Queries spread inside a block by eps around qbar, keys constant per
    block: the block-level correction's error is first order in eps (halving
    eps halves it) while the per-row correction is exact. Keys spread by eps
    with values constant per block: the per-row error is second order
    (App. B: the denominator error is second order in the centred spread)."""
    rng = np.random.default_rng(8)
    N, d = 256, 4

    def centred(a):
        return a - np.repeat(a.reshape(N // 64, 64, d).mean(axis=1), 64, axis=0)

    base_q = np.repeat(rand(rng, N // 64, d), 64, axis=0)
    uq, uk = centred(rand(rng, N, d)), centred(rand(rng, N, d))
    kb = np.repeat(rand(rng, N // 64, d), 64, axis=0)
    v = rand(rng, N, d)
    vb = np.repeat(rand(rng, N // 64, d), 64, axis=0)
    keep = np.zeros((N // 64, N // 64), dtype=bool)
    keep[:, 0] = True

    def err(q, k, vv, row):
        r = attend_head(q, k, vv, 64, 64, 0.0, keep_override=keep, row_correction=row)
        return np.abs(r["out"] - sdpa64(q, k, vv)).max()

    blk = [err(base_q + e * uq, kb, v, False) for e in (0.02, 0.01)]
    assert blk[0] / blk[1] == pytest.approx(2.0, rel=0.05)
    assert max(err(base_q + e * uq, kb, v, True) for e in (0.02, 0.01)) < 1e-13
    row = [err(base_q, kb + e * uk, vb, True) for e in (0.02, 0.01)]
    assert row[0] / row[1] == pytest.approx(4.0, rel=0.05)
