"""Shared parity machinery for the GPU tests: run the HIP path through the C
ABI, run the fp64 oracle on the same bf16 inputs, compare.

Tolerances:
  * kept-block bitmap: exact, except blocks whose fp64 proxy lies within 1e-3
    of the threshold (M_i - tau, or mean_i + beta std_i for the Gaussian
    rule; either decision is correct there); forced sink blocks exactly kept;
  * output: max |gpu - oracle| <= 2e-2 with the oracle conditioned on the
    GPU's routing (bf16 inputs, fp32 accumulation, unit-scale outputs);
  * stats: exact integer agreement with the exported bitmap.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np
import torch

import block_sparse_attention_14_amd as sa
from oracle import attend_head, block_means, gauss_threshold, gauss_threshold_diag, proxy_scores, route
from workloads import bf16_bits_to_f64

BITMAP_TIE = 1e-3
OUT_ATOL = 2e-2


def to_device_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def run_gpu(qb, kb, vb, tau, flags=0, runner: Optional[sa.SolAttention] = None, device="cuda", beta=None,
            sinks=None, diag=False):
    """Returns (out fp32 numpy, keep bool [B,H,Nq,Nk], stats dict)."""
    B, H, N, d = qb.shape
    q, k, v = (to_device_bf16(x, device) for x in (qb, kb, vb))
    runner = runner or sa.SolAttention(B, H, N, d, device)
    bm = torch.zeros(sa.bitmap_shape(B, H, N), dtype=torch.int32, device=device)
    out = runner(q, k, v, tau, flags=flags, bitmap=bm, beta=beta, sinks=sinks, diag=diag)
    torch.cuda.synchronize()
    keep = sa.unpack_bitmap(bm, -(-N // 64))
    return out.cpu().numpy(), keep, runner.read_stats()


def oracle_route(q, k, tau, beta=None, sinks=None, diag=False):
    """fp64 proxy scores, thresholds, keep mask and the forced-sink mask of one head."""
    d = q.shape[1]
    qbar, _ = block_means(q, 64)
    kbar, _ = block_means(k, 64)
    s = proxy_scores(qbar, kbar, d)
    if beta is None:
        M, keep = route(s, tau)
        theta = M - tau
    else:
        theta = (gauss_threshold_diag if diag else gauss_threshold)(qbar, kbar, d, beta)
        keep = s >= theta[:, None]
    forced = np.zeros_like(keep)
    if sinks is not None and sinks[1] > 0:
        forced[:, sinks[0]:sinks[0] + sinks[1]] = True
    return s, theta, keep | forced, forced


def check_bitmap(gpu_keep: np.ndarray, s: np.ndarray, theta: np.ndarray, keep: np.ndarray, forced: np.ndarray,
                 rowmax: bool, where=""):
    if not np.isfinite(theta).any() and rowmax:
        assert gpu_keep.all(), f"{where}: tau=inf must keep every block"
        return
    assert gpu_keep[forced].all(), f"{where}: a forced sink block was not kept"
    near = (np.abs(s - theta[:, None]) <= BITMAP_TIE) & ~forced
    bad = (gpu_keep != keep) & ~near
    assert not bad.any(), f"{where}: {int(bad.sum())} routing decisions differ away from the threshold, " \
                          f"first at {np.argwhere(bad)[:3].tolist()}"
    if rowmax:
        assert gpu_keep.sum(axis=1).min() >= 1, f"{where}: a query block kept nothing"
    # every kept block is forced, or within the tie band of the threshold, or above it
    above = s >= theta[:, None] - BITMAP_TIE
    assert (above | forced)[gpu_keep].all()


def check_head(qb, kb, vb, out_gpu, keep_gpu, tau, query_blocks: Optional[Iterable[int]] = None, where="",
               beta=None, sinks=None, row_correction=False, diag=False, correction=True):
    """Bitmap on every query block of the head; outputs on `query_blocks` (all if None).
    correction=False: the exact-only ablation (skipped blocks dropped)."""
    q, k, v = (bf16_bits_to_f64(x) for x in (qb, kb, vb))
    s, theta, keep, forced = oracle_route(q, k, tau, beta, sinks, diag)
    check_bitmap(keep_gpu, s, theta, keep, forced, beta is None, where)
    r = attend_head(q, k, v, 64, 64, tau, keep_override=keep_gpu, query_blocks=query_blocks,
                    row_correction=row_correction, correction=correction)
    rows = np.concatenate([np.arange(i * 64, min(q.shape[0], i * 64 + 64)) for i in r["rows"]])
    err = np.abs(out_gpu[rows] - r["out"][rows]).max()
    assert np.isfinite(out_gpu[rows]).all(), f"{where}: non-finite output"
    assert err <= OUT_ATOL, f"{where}: max abs error {err:.3e} > {OUT_ATOL}"
    return err


def check_stats(stats, keep_all: np.ndarray, N: int):
    """keep_all: [B, H, Nq, Nk] bool from the bitmap."""
    Nq, Nk = keep_all.shape[-2:]
    n = np.minimum(64, N - 64 * np.arange(Nk)).astype(np.int64)
    per = keep_all.sum(axis=-1)
    assert stats["kept_blocks"] == int(keep_all.sum())
    assert stats["total_blocks"] == int(np.prod(keep_all.shape))
    assert stats["min_kept"] == int(per.min()) and stats["max_kept"] == int(per.max())
    pairs = (keep_all * n[None, None, None, :]).sum(axis=-1) * n[None, None, :]  # n_i == n_j sizes
    assert stats["kept_pairs"] == int(pairs.sum())


QUEUES = 8  # the fused kernel's work queues, one per XCD, each over a contiguous range of items


def stratified_blocks(B: int, H: int, Nq: int, rng: np.random.Generator, per_queue: int = 3):
    """Query blocks to check on a layer too large for the oracle to run whole,
    chosen where scheduling could go wrong: in each of the eight queue ranges
    of work items (an item is a pair of neighbouring query blocks, numbered
    head-major), the first two and last two items (where workgroups begin and
    where stealing from a drained queue starts), the item that opens the last
    third (where a planned order switches to heaviest first), and `per_queue`
    random items of that last third and of the first two thirds; plus the
    first and the ragged last query block of every head.
    Returns {(b, h): sorted list of query blocks}."""
    npairs = (Nq + 1) // 2
    nitems = B * H * npairs
    items = set()
    for x in range(QUEUES):
        lo, hi = x * nitems // QUEUES, (x + 1) * nitems // QUEUES
        if hi <= lo:
            continue
        tail = lo + 2 * (hi - lo) // 3
        items.update(i for i in (lo, lo + 1, hi - 2, hi - 1, tail) if lo <= i < hi)
        if hi > tail:
            items.update(rng.integers(tail, hi, size=per_queue).tolist())
        if tail > lo:
            items.update(rng.integers(lo, tail, size=per_queue).tolist())
    picks = {(b, h): {0, Nq - 1} for b in range(B) for h in range(H)}
    for it in items:
        bh, p = divmod(it, npairs)
        blocks = picks[(bh // H, bh % H)]
        blocks.add(2 * p)
        if 2 * p + 1 < Nq:
            blocks.add(2 * p + 1)
    return {key: sorted(v) for key, v in picks.items()}


def sample_blocks(Nq: int, rng: np.random.Generator, k: int = 6) -> Sequence[int]:
    """First, last (ragged) and a few random query blocks."""
    picks = {0, Nq - 1}
    picks.update(rng.choice(Nq, size=min(k, Nq), replace=False).tolist())
    return sorted(picks)
