"""Seeded, synthetic, video-DiT-shaped attention inputs.

The Sol-Attn pages (paperlayer.ai summary of arXiv 2607.24027, section 4 and
appendix A) evaluate on Wan2.1-14B, HunyuanVideo-13B, Bernini-14B, Ideogram 4
and SANA-WM. None of those weights or prompts are available, so these
generators stand in for their self-attention inputs: tokens are patches of a
(t, h, w) latent grid in row-major order, q/k/v are standard normal per head,
and a 3-D sinusoidal position code (scaled by 3) is added to q and k so that
neighbouring tokens attend to each other the way video-DiT heads do.

Every array is drawn from ``numpy.random.PCG64(SeedSequence([seed, b, h]))``,
so any single head can be regenerated on its own. bf16 inputs are rounded from
float32 with round-to-nearest-even on the bit pattern, which is the rounding
the GPU receives and the oracle up-casts exactly.

Nothing in this module computes any part of the attention method.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Iterable, Optional, Sequence, Tuple

import numpy as np

INF = math.inf


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic attention layer: shapes, taus, construction knobs."""

    name: str
    B: int
    H: int
    grid: Tuple[int, int, int]  # (t, h, w) latent grid, tokens in row-major order
    d: int
    dtype: str  # "fp32" (rounded once to bf16 for the GPU) or "bf16"
    taus: Tuple[float, ...]
    seed: int
    Bq: int = 64
    Bk: int = 64
    # per-head scale of the position code added to q and k
    locality: Tuple[float, ...] = ()
    # heads whose first `sink_blocks` KV blocks get k += 2 * mean_t(q)
    sink_heads: Tuple[int, ...] = ()
    sink_blocks: int = 0
    # scale of the position code added to v (0: values independent per token)
    value_locality: float = 0.0
    # scale of the per-token N(0, 1) draws of q and k (1: unit noise)
    qk_noise: float = 1.0
    description: str = ""

    @property
    def N(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def Nq(self) -> int:
        return -(-self.N // self.Bq)

    @property
    def Nk(self) -> int:
        return -(-self.N // self.Bk)

    def head_locality(self, h: int) -> float:
        if self.locality:
            return float(self.locality[h])
        return 3.0

    def dense_flops(self) -> float:
        """4*B*H*N^2*d: both GEMMs of dense non-causal attention."""
        return 4.0 * self.B * self.H * float(self.N) ** 2 * self.d


def _wl(**kw) -> Workload:
    return Workload(**kw)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        _wl(
            name="tiny_fp32",
            B=1, H=2, grid=(4, 16, 16), d=64, dtype="fp32",
            taus=(0.0, 2.0, 4.0, INF), seed=1000,
            description="tiny fp32 layer, 4x16x16 grid, N=1024, d=64",
        ),
        _wl(
            name="image_dit_4k",
            B=2, H=24, grid=(1, 64, 64), d=128, dtype="bf16",
            taus=(2.0, 4.0, 8.0), seed=1001,
            description="image-DiT layer, 64x64 grid, N=4096, d=128",
        ),
        _wl(
            name="video_dit_32k",
            B=1, H=12, grid=(21, 30, 52), d=128, dtype="bf16",
            taus=(2.0, 4.0, 8.0, INF), seed=1002,
            description="video-DiT layer, 21x30x52 grid, N=32760 (last block 56), d=128",
        ),
        _wl(
            name="video_dit_32k_imbalance",
            B=1, H=12, grid=(21, 30, 52), d=128, dtype="bf16",
            taus=(8.0,), seed=1003,
            locality=(3.0,) * 6 + (0.0,) * 6,
            sink_heads=(0, 1), sink_blocks=4,
            description=("budget-imbalance video-DiT layer, N=32760, heads 0-5 local, "
                         "6-11 diffuse, 4 sink KV blocks on heads 0-1"),
        ),
        _wl(
            name="video_dit_32k_smoothv",
            B=1, H=12, grid=(21, 30, 52), d=128, dtype="bf16",
            taus=(2.0, 4.0, 8.0), seed=1005, value_locality=3.0,
            description=("video-DiT layer, N=32760, values sharing the position code "
                         "(spatially smooth), for the correction ablation"),
        ),
        _wl(
            name="video_dit_32k_mild",
            B=1, H=12, grid=(21, 30, 52), d=128, dtype="bf16",
            taus=(1.0, 2.0, 4.0), seed=1006, locality=(1.5,) * 12, qk_noise=0.5, value_locality=3.0,
            description=("video-DiT layer, N=32760, milder locality (1.5 P(pos) on q and k, per-token "
                         "draws of q and k at half scale) and smooth values: skipped blocks hold a "
                         "share of the attention mass that the correction can recover"),
        ),
        _wl(
            name="video_dit_119k",
            B=1, H=24, grid=(33, 45, 80), d=128, dtype="bf16",
            taus=(2.0, 4.0, 8.0), seed=1004,
            description="large video-DiT layer, 33x45x80 grid, N=118800 (last block 16), d=128",
        ),
    ]
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


# --------------------------------------------------------------------------
# position code
# --------------------------------------------------------------------------

def _axis_code(pos: np.ndarray, m: int) -> np.ndarray:
    """Interleaved (sin, cos) pairs of one axis, frequencies 10000^(-2i/m)."""
    i = np.arange(m // 2, dtype=np.float64)
    omega = 10000.0 ** (-2.0 * i / m)
    ang = pos[:, None].astype(np.float64) * omega[None, :]
    out = np.empty((pos.shape[0], m), dtype=np.float64)
    out[:, 0::2] = np.sin(ang)
    out[:, 1::2] = np.cos(ang)
    return out


def pos_code(grid: Tuple[int, int, int], d: int) -> np.ndarray:
    """3-D sinusoidal code over a (t, h, w) grid, one row per token, norm sqrt(d).

    d is split into contiguous groups d_t = d_h = 2*floor(d/6) and
    d_w = d - d_t - d_h (64 -> 20/20/24, 128 -> 42/42/44); each group holds the
    code of one axis; each token's row is then rescaled to L2 norm sqrt(d).
    """
    T, Hh, W = grid
    dt = dh = 2 * (d // 6)
    dw = d - dt - dh
    assert dw > 0 and dw % 2 == 0
    t, h, w = np.meshgrid(np.arange(T), np.arange(Hh), np.arange(W), indexing="ij")
    t, h, w = t.ravel(), h.ravel(), w.ravel()
    P = np.concatenate([_axis_code(t, dt), _axis_code(h, dh), _axis_code(w, dw)], axis=1)
    P *= math.sqrt(d) / np.linalg.norm(P, axis=1, keepdims=True)
    return P


# --------------------------------------------------------------------------
# bf16 bit conversion (data plumbing, not arithmetic of the method)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 -> bf16 with round-to-nearest-even; returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    return bf16_bits_to_f32(bits).astype(np.float64)


# --------------------------------------------------------------------------
# per-head generation
# --------------------------------------------------------------------------

_POS_CACHE: Dict[Tuple[Tuple[int, int, int], int], np.ndarray] = {}


def _pos32(grid, d) -> np.ndarray:
    key = (tuple(grid), d)
    if key not in _POS_CACHE:
        _POS_CACHE.clear()
        _POS_CACHE[key] = pos_code(grid, d).astype(np.float32)
    return _POS_CACHE[key]


def make_head(wl: Workload, b: int, h: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """float32 q, k, v of head (b, h), each [N, d], before any bf16 rounding."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, b, h])))
    N, d = wl.N, wl.d
    q = rng.standard_normal((N, d), dtype=np.float32)
    k = rng.standard_normal((N, d), dtype=np.float32)
    v = rng.standard_normal((N, d), dtype=np.float32)
    if wl.qk_noise != 1.0:
        q *= np.float32(wl.qk_noise)
        k *= np.float32(wl.qk_noise)
    alpha = wl.head_locality(h)
    if alpha != 0.0:
        P = _pos32(wl.grid, d)
        q += np.float32(alpha) * P
        k += np.float32(alpha) * P
    if wl.value_locality != 0.0:
        v += np.float32(wl.value_locality) * _pos32(wl.grid, d)
    if h in wl.sink_heads and wl.sink_blocks > 0:
        shift = (2.0 * q.astype(np.float64).mean(axis=0)).astype(np.float32)
        k[: wl.sink_blocks * wl.Bk] += shift[None, :]
    return q, k, v


def make_inputs(
    wl: Workload,
    heads: Optional[Iterable[Tuple[int, int]]] = None,
    keep_fp32: bool = False,
) -> Dict[str, np.ndarray]:
    """All heads (or the listed (b, h) heads) as bf16 bit arrays [B, H, N, d].

    Returns {"q", "k", "v"} as uint16 bf16 bits; with keep_fp32 also
    {"q32", "k32", "v32"} holding the unrounded float32 values. Heads not
    listed are left zero.
    """
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    out = {n: np.zeros((B, H, N, d), dtype=np.uint16) for n in ("q", "k", "v")}
    if keep_fp32:
        out.update({n + "32": np.zeros((B, H, N, d), dtype=np.float32) for n in ("q", "k", "v")})
    todo: Sequence[Tuple[int, int]] = (
        list(heads) if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    )
    for b, h in todo:
        arrs = make_head(wl, b, h)
        for n, a in zip(("q", "k", "v"), arrs):
            out[n][b, h] = f32_to_bf16_bits(a)
            if keep_fp32:
                out[n + "32"][b, h] = a
    return out
