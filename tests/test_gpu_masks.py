"""GPU routers without attention (sol_attn_mask_*) against the forward's own
routing and the fp64 oracle's top-k / top-p masks.

Bars: the threshold router reproduces the bitmap of sol_attn_forward_debug bit
for bit (same arithmetic); top-k keeps exactly min(k, Nk) blocks per row that
form a top set of the fp64 scores up to 1e-3; top-p keeps a top set whose
size lies between the oracle's sizes at p - 1e-4 and p + 1e-4.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_14_amd as sa
from oracle import block_means, proxy_scores, topk_mask, topp_mask
from workloads import Workload, bf16_bits_to_f64, get_workload, make_inputs

from parity import check_bitmap, oracle_route, to_device_bf16

pytestmark = pytest.mark.gpu

TIE = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sa.lib()


def _custom(N, d, H=2, seed=31):
    return Workload(name=f"custom_N{N}_d{d}", B=1, H=H, grid=(1, 1, N), d=d, dtype="bf16", taus=(), seed=seed)


def _setup(wl):
    x = make_inputs(wl)
    q, k, v = (to_device_bf16(x[n]) for n in "qkv")
    kpool, vmean = sa.pool(k, v)
    return x, q, k, v, kpool, vmean


def _scores(x, b, h):
    q, k = bf16_bits_to_f64(x["q"][b, h]), bf16_bits_to_f64(x["k"][b, h])
    qbar, _ = block_means(q, 64)
    kbar, _ = block_means(k, 64)
    return proxy_scores(qbar, kbar, q.shape[1])


def _check_top_set(s, keep, where):
    for i in range(s.shape[0]):
        kept, dropped = s[i, keep[i]], s[i, ~keep[i]]
        if len(kept) and len(dropped):
            assert kept.min() >= dropped.max() - TIE, f"{where} row {i}: not a top set"


WLS = [("tiny_fp32", None), ("custom", (1000, 128)), ("custom", (130, 64)), ("image_dit_4k", None)]


def _wl(name, arg):
    return get_workload(name) if arg is None else _custom(*arg)


@pytest.mark.parametrize("name,arg", WLS)
@pytest.mark.parametrize("route", [dict(tau=0.0), dict(tau=2.0), dict(tau=8.0), dict(tau=math.inf),
                                   dict(tau=1.0, sinks=(1, 2)), dict(tau=0.0, sinks=(0, 1))])
def test_threshold_router_matches_forward_and_oracle(name, arg, route):
    wl = _wl(name, arg)
    x, q, k, v, kpool, _ = _setup(wl)
    mb = sa.MaskBuilder(wl.B, wl.H, wl.N, wl.d)
    got = mb.threshold(q, kpool, **route).clone()
    fwd = sa.SolAttention(wl.B, wl.H, wl.N, wl.d)
    bm = torch.zeros_like(got)
    fwd(q, k, v, route.get("tau", 0.0), bitmap=bm, beta=route.get("beta"), sinks=route.get("sinks"))
    torch.cuda.synchronize()
    assert torch.equal(got, bm), "threshold router and forward routed differently"
    keep = sa.unpack_bitmap(got, wl.Nk)
    for b in range(wl.B):
        for h in range(wl.H):
            qh, kh = bf16_bits_to_f64(x["q"][b, h]), bf16_bits_to_f64(x["k"][b, h])
            s, theta, ok, forced = oracle_route(qh, kh, route.get("tau", 0.0), route.get("beta"), route.get("sinks"))
            check_bitmap(keep[b, h], s, theta, ok, forced, "beta" not in route, where=f"{wl.name} b={b} h={h}")


def test_threshold_router_rejects_gaussian_rules():
    """The Gaussian thresholds take their pooled-key statistics from the
    forward's workspace, which the mask router does not have."""
    import ctypes

    from block_sparse_attention_14_amd import _lib

    wl = _custom(1000, 128, H=1)
    x, q, k, v, kpool, _ = _setup(wl)
    bm = torch.zeros(sa.bitmap_shape(1, 1, 1000), dtype=torch.int32, device=q.device)
    for rule in (sa.SOL_ROUTE_GAUSS, sa.SOL_ROUTE_GAUSS_DIAG):
        route = _lib.sol_attn_route(rule, 0.0, 1.0, 0, 0)
        ws = torch.empty(sa.lib().sol_attn_mask_workspace_bytes(1, 1, 1000, 128, 64, 64) // 8 + 1, dtype=torch.int64,
                         device=q.device)
        rc = sa.lib().sol_attn_mask_threshold(q.data_ptr(), kpool.data_ptr(), 1, 1, 1000, 128, 64, 64,
                                              ctypes.byref(route), bm.data_ptr(), ws.data_ptr(), ws.numel() * 8, None)
        assert rc == sa.SOL_EUNSUPPORTED


@pytest.mark.parametrize("name,arg", WLS)
@pytest.mark.parametrize("kk", [0, 1, 5, 16, 10_000])
def test_topk_router(name, arg, kk):
    wl = _wl(name, arg)
    x, q, k, v, kpool, _ = _setup(wl)
    keep = sa.unpack_bitmap(sa.MaskBuilder(wl.B, wl.H, wl.N, wl.d).topk(q, kpool, kk), wl.Nk)
    for b in range(wl.B):
        for h in range(wl.H):
            s = _scores(x, b, h)
            assert (keep[b, h].sum(axis=1) == min(kk, wl.Nk)).all()
            _check_top_set(s, keep[b, h], f"{wl.name} k={kk}")
            exact = topk_mask(s, kk)
            gap = np.sort(s, axis=1)[:, ::-1]
            if 0 < kk < wl.Nk:  # away from near-ties the sets are identical
                clear = (gap[:, kk - 1] - gap[:, kk]) > TIE
                assert (keep[b, h][clear] == exact[clear]).all()


def _topp_bounds(s, p, delta=1e-4):
    lo = topp_mask(s, p - delta).sum(axis=1)
    hi = topp_mask(s, p + delta).sum(axis=1)
    return lo, hi


@pytest.mark.parametrize("name,arg", WLS)
@pytest.mark.parametrize("pp", [0.0, 0.3, 0.9, 0.99, 1.0])
def test_topp_router(name, arg, pp):
    wl = _wl(name, arg)
    x, q, k, v, kpool, _ = _setup(wl)
    keep = sa.unpack_bitmap(sa.MaskBuilder(wl.B, wl.H, wl.N, wl.d).topp(q, kpool, pp), wl.Nk)
    for b in range(wl.B):
        for h in range(wl.H):
            s = _scores(x, b, h)
            _check_top_set(s, keep[b, h], f"{wl.name} p={pp}")
            n = keep[b, h].sum(axis=1)
            lo, hi = _topp_bounds(s, pp)
            assert ((n >= lo) & (n <= hi)).all(), f"{wl.name} p={pp}: kept counts outside the oracle's range"
            if pp >= 1.0:
                assert keep[b, h].all()
            if pp <= 0.0:
                assert (n == 1).all()


def test_routers_on_the_video_layer():
    wl = get_workload("video_dit_32k")
    x, q, k, v, kpool, _ = _setup(wl)
    mb = sa.MaskBuilder(wl.B, wl.H, wl.N, wl.d)
    fwd = sa.SolAttention(wl.B, wl.H, wl.N, wl.d)
    bm = torch.zeros(sa.bitmap_shape(wl.B, wl.H, wl.N), dtype=torch.int32, device=q.device)
    fwd(q, k, v, 8.0, bitmap=bm)
    assert torch.equal(mb.threshold(q, kpool, tau=8.0), bm)
    kk = 24
    keep_k = sa.unpack_bitmap(mb.topk(q, kpool, kk), wl.Nk)
    keep_p = sa.unpack_bitmap(mb.topp(q, kpool, 0.9), wl.Nk)
    for h in (0, 7, 11):
        s = _scores(x, 0, h)
        assert (keep_k[0, h].sum(axis=1) == kk).all()
        _check_top_set(s, keep_k[0, h], "topk")
        _check_top_set(s, keep_p[0, h], "topp")
        lo, hi = _topp_bounds(s, 0.9)
        n = keep_p[0, h].sum(axis=1)
        assert ((n >= lo) & (n <= hi)).all()
