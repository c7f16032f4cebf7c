"""Python binding of the Sol-Attn C ABI.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, then their device pointers and torch's current HIP stream go to
libsolattn.so, whose kernels do all of the work. torch provides the device
memory and the stream; nothing here computes any part of the attention.
"""
from __future__ import annotations

import ctypes
import math
from typing import Dict, Optional, Tuple

import torch

from . import _lib
from ._lib import (SOL_F_EXACT_ONLY, SOL_F_GROUP2, SOL_F_GROUP4, SOL_F_GROUP6, SOL_F_GROUP8,  # noqa: F401
                   SOL_F_GROUP16, SOL_F_OUT_BF16, SOL_F_PLANNED, SOL_F_POOLED, SOL_F_PREPARED,  # noqa: F401
                   SOL_F_ROW_CORRECTION, check, lib)  # noqa: F401

STATS_WORDS = 4  # sol_attn_stats is 32 bytes


def group_flag(group: int) -> int:
    """The SOL_F_GROUP* bits for 2, 4, 6, 8 or 16 query blocks per work item (0: automatic)."""
    try:
        return {0: 0, 2: SOL_F_GROUP2, 4: SOL_F_GROUP4, 6: SOL_F_GROUP6, 8: SOL_F_GROUP8, 16: SOL_F_GROUP16}[int(group)]
    except KeyError:
        raise ValueError("group must be 0, 2, 4, 6, 8 or 16") from None


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check_qkv(name: str, t: torch.Tensor, shape=None) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16, got {t.dtype}")
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, H, N, d], got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_f32(name: str, t: torch.Tensor, shape, device) -> None:
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape) or t.device != device:
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {tuple(shape)} on {device}")


def _device(device) -> torch.device:
    dev = torch.device(device)
    return torch.device("cuda", torch.cuda.current_device()) if dev.index is None else dev


def workspace_bytes(B: int, H: int, N: int, d: int, Bq: int = 64, Bk: int = 64) -> int:
    return int(lib().sol_attn_workspace_bytes(B, H, N, d, Bq, Bk))


def pooled_shape(B: int, H: int, N: int, d: int, Bk: int = 64) -> Tuple[int, int, int, int]:
    return (B, H, -(-N // Bk), d)


def bitmap_shape(B: int, H: int, N: int, Bq: int = 64, Bk: int = 64) -> Tuple[int, int, int, int]:
    return (B, H, -(-N // Bq), -(-(-(-N // Bk)) // 32))


def new_stats(device) -> torch.Tensor:
    return torch.zeros(STATS_WORDS, dtype=torch.int64, device=device)


def read_stats(t: torch.Tensor) -> Dict[str, int]:
    """Decode a stats tensor written by forward() (synchronises)."""
    raw = t.detach().cpu().numpy().tobytes()
    s = _lib.sol_attn_stats.from_buffer_copy(raw)
    return {f: int(getattr(s, f)) for f, _ in _lib.sol_attn_stats._fields_}


def pool(k: torch.Tensor, v: torch.Tensor, Bk: int = 64,
         kpool: Optional[torch.Tensor] = None, vmean: Optional[torch.Tensor] = None):
    """Per-block means of k and v (fp32, [B, H, ceil(N/Bk), d])."""
    _check_qkv("k", k)
    _check_qkv("v", v, k.shape)
    B, H, N, d = k.shape
    ps = pooled_shape(B, H, N, d, Bk)
    kpool = torch.empty(ps, dtype=torch.float32, device=k.device) if kpool is None else kpool
    vmean = torch.empty(ps, dtype=torch.float32, device=k.device) if vmean is None else vmean
    _check_f32("kpool", kpool, ps, k.device)
    _check_f32("vmean", vmean, ps, k.device)
    rc = lib().sol_attn_pool(_ptr(k), _ptr(v), _ptr(kpool), _ptr(vmean), B, H, N, d, Bk, _stream(k.device))
    check(rc, "sol_attn_pool")
    return kpool, vmean


class SolAttention:
    """Reusable buffers (pooled k/v, workspace, stats) for one [B, H, N, d] shape.

    Calling the object runs the pooling pre-pass and the fused forward on the
    current stream and returns the fp32 output.
    """

    def __init__(self, B: int, H: int, N: int, d: int, device="cuda", Bq: int = 64, Bk: int = 64):
        self.B, self.H, self.N, self.d, self.Bq, self.Bk = B, H, N, d, Bq, Bk
        self.device = _device(device)
        nbytes = workspace_bytes(B, H, N, d, Bq, Bk)
        if nbytes == 0:
            rc = _lib.SOL_EUNSUPPORTED if d > 0 and N > 0 and B > 0 and H > 0 else _lib.SOL_EINVAL
            check(rc, "sol_attn_workspace_bytes")
        ps = pooled_shape(B, H, N, d, Bk)
        self.kpool = torch.empty(ps, dtype=torch.float32, device=self.device)
        self.vmean = torch.empty(ps, dtype=torch.float32, device=self.device)
        self.workspace = torch.zeros(-(-nbytes // 8), dtype=torch.int64, device=self.device)
        assert self.workspace.data_ptr() % 256 == 0
        self.stats = new_stats(self.device)

    def __call__(self, q, k, v, tau: float, flags: int = 0, out: Optional[torch.Tensor] = None,
                 stats: bool = True, bitmap: Optional[torch.Tensor] = None, beta: Optional[float] = None,
                 sinks: Optional[Tuple[int, int]] = None, diag: bool = False,
                 out_dtype: torch.dtype = torch.float32, group: int = 0) -> torch.Tensor:
        """Forward on the current stream. ``tau`` is the row-max offset; with
        ``beta`` set, the Gaussian-calibrated rule (mean + beta * std of each
        proxy row) routes instead and ``tau`` is ignored; ``diag`` selects its
        diagonal estimator from the pooled-key statistics. ``sinks`` =
        (first, count) key blocks that are always kept. The output is fp32,
        or bf16 (SOL_F_OUT_BF16) when ``out`` or ``out_dtype`` is bfloat16.
        ``group`` (2, 4, 6, 8 or 16; 0 = the library's choice) sets the query
        blocks per work item (SOL_F_GROUP*)."""
        flags |= group_flag(group)
        shape = (self.B, self.H, self.N, self.d)
        _check_qkv("q", q, shape)
        _check_qkv("k", k, shape)
        _check_qkv("v", v, shape)
        if q.device != self.device or k.device != self.device or v.device != self.device:
            raise ValueError(f"q, k, v must be on {self.device}")
        if out is None:
            if out_dtype not in (torch.float32, torch.bfloat16):
                raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")
            out = torch.empty(shape, dtype=out_dtype, device=self.device)
        if out.dtype == torch.bfloat16:
            flags |= SOL_F_OUT_BF16
            if not out.is_contiguous() or tuple(out.shape) != shape or out.device != self.device:
                raise ValueError(f"out must be a contiguous tensor of shape {shape} on {self.device}")
        else:
            if flags & SOL_F_OUT_BF16:
                raise ValueError("SOL_F_OUT_BF16 needs a bfloat16 out tensor")
            _check_f32("out", out, shape, self.device)
        bm_ptr = None
        if bitmap is not None:
            bs = bitmap_shape(self.B, self.H, self.N, self.Bq, self.Bk)
            if bitmap.dtype != torch.int32 or tuple(bitmap.shape) != bs or not bitmap.is_contiguous() \
                    or bitmap.device != self.device:
                raise ValueError(f"bitmap must be a contiguous int32 tensor of shape {bs} on {self.device}")
            bm_ptr = _ptr(bitmap)
        if beta is not None or sinks is not None:
            rule = _lib.SOL_ROUTE_ROWMAX if beta is None else (
                _lib.SOL_ROUTE_GAUSS_DIAG if diag else _lib.SOL_ROUTE_GAUSS)
            route = _lib.sol_attn_route(
                rule,
                float(tau) if beta is None else 0.0, 0.0 if beta is None else float(beta),
                0 if sinks is None else int(sinks[0]), 0 if sinks is None else int(sinks[1]))
            rc = lib().sol_attn_forward_ex(
                _ptr(q), _ptr(k), _ptr(v), _ptr(out), self.B, self.H, self.N, self.d, self.Bq, self.Bk,
                ctypes.byref(route), ctypes.c_uint(flags), _ptr(self.stats) if stats else None,
                _ptr(self.kpool), _ptr(self.vmean), _ptr(self.workspace), self.workspace.numel() * 8,
                _stream(self.device), bm_ptr)
            check(rc, "sol_attn_forward_ex")
            return out
        args = (
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), self.B, self.H, self.N, self.d, self.Bq, self.Bk,
            ctypes.c_float(float(tau)), ctypes.c_uint(flags), _ptr(self.stats) if stats else None,
            _ptr(self.kpool), _ptr(self.vmean), _ptr(self.workspace), self.workspace.numel() * 8,
            _stream(self.device),
        )
        if bitmap is None:
            rc = lib().sol_attn_forward(*args)
            check(rc, "sol_attn_forward")
        else:
            rc = lib().sol_attn_forward_debug(*args, bm_ptr)
            check(rc, "sol_attn_forward_debug")
        return out

    def plan(self, q: torch.Tensor, tau: float) -> None:
        """Item costs and the planned order (per queue: first two thirds in
        sequence, last third heaviest first) into the workspace, for forwards
        with SOL_F_PLANNED (needs self.kpool to hold the pooled keys, e.g. from
        pool())."""
        _check_qkv("q", q, (self.B, self.H, self.N, self.d))
        rc = lib().sol_attn_plan(_ptr(q), _ptr(self.kpool), self.B, self.H, self.N, self.d, self.Bq, self.Bk,
                                 ctypes.c_float(float(tau)), _ptr(self.workspace), self.workspace.numel() * 8,
                                 _stream(self.device))
        check(rc, "sol_attn_plan")

    def prepare(self, q: torch.Tensor, flags: int = 0) -> None:
        """The forward's pre-pass (pooled queries, routing planes of self.kpool
        and self.vmean) into the workspace, for forwards with SOL_F_PREPARED;
        flags: 0 or SOL_F_ROW_CORRECTION."""
        _check_qkv("q", q, (self.B, self.H, self.N, self.d))
        rc = lib().sol_attn_prepare(_ptr(q), _ptr(self.kpool), _ptr(self.vmean), self.B, self.H, self.N, self.d,
                                    self.Bq, self.Bk, ctypes.c_uint(int(flags)), _ptr(self.workspace),
                                    self.workspace.numel() * 8, _stream(self.device))
        check(rc, "sol_attn_prepare")

    def read_stats(self) -> Dict[str, int]:
        return read_stats(self.stats)


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tau: float, Bq: int = 64, Bk: int = 64,
            flags: int = 0, return_bitmap: bool = False, return_stats: bool = False,
            beta: Optional[float] = None, sinks: Optional[Tuple[int, int]] = None,
            out_dtype: torch.dtype = torch.float32):
    """One-shot sparse attention forward (allocates its buffers).

    Returns out (fp32, or bf16 with ``out_dtype``), plus the kept-block bitmap [B, H, Nq, ceil(Nk/32)]
    (int32 words) and/or the stats dict when asked.
    """
    _check_qkv("q", q)
    B, H, N, d = q.shape
    if beta is None and (math.isnan(tau) or tau < 0):
        check(_lib.SOL_EINVAL, "sol_attn_forward")
    runner = SolAttention(B, H, N, d, q.device, Bq, Bk)
    bm = None
    if return_bitmap:
        bm = torch.zeros(bitmap_shape(B, H, N, Bq, Bk), dtype=torch.int32, device=q.device)
    out = runner(q, k, v, tau, flags=flags, bitmap=bm, beta=beta, sinks=sinks, out_dtype=out_dtype)
    res = [out]
    if return_bitmap:
        res.append(bm)
    if return_stats:
        res.append(runner.read_stats())
    return res[0] if len(res) == 1 else tuple(res)


def forward_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, tau: float = 0.0,
                    flags: int = 0, stats: Optional[torch.Tensor] = None, bitmap: Optional[torch.Tensor] = None,
                    beta: Optional[float] = None, sinks: Optional[Tuple[int, int]] = None,
                    diag: bool = False) -> torch.Tensor:
    """sol_attn_forward_noalloc: the forward with its pooled buffers and
    workspace in the library's static device scratch array, so nothing is
    allocated, by torch or the library (the caller passes ``out`` and, if
    wanted, ``stats`` (new_stats()) and ``bitmap``). Routing as for
    SolAttention.__call__. Calls that overlap on one GPU race."""
    _check_qkv("q", q)
    shape = tuple(q.shape)
    _check_qkv("k", k, shape)
    _check_qkv("v", v, shape)
    B, H, N, d = shape
    if k.device != q.device or v.device != q.device or out.device != q.device:
        raise ValueError("q, k, v and out must be on one device")
    if not out.is_contiguous() or tuple(out.shape) != shape:
        raise ValueError(f"out must be a contiguous tensor of shape {shape}")
    if out.dtype == torch.bfloat16:
        flags |= SOL_F_OUT_BF16
    elif out.dtype != torch.float32:
        raise ValueError("out must be float32 or bfloat16")
    if stats is not None and (stats.dtype != torch.int64 or stats.numel() != STATS_WORDS or stats.device != q.device):
        raise ValueError("stats must come from new_stats() on the inputs' device")
    if bitmap is not None:
        bs = bitmap_shape(B, H, N)
        if bitmap.dtype != torch.int32 or tuple(bitmap.shape) != bs or not bitmap.is_contiguous() \
                or bitmap.device != q.device:
            raise ValueError(f"bitmap must be a contiguous int32 tensor of shape {bs} on {q.device}")
    rule = _lib.SOL_ROUTE_ROWMAX if beta is None else (_lib.SOL_ROUTE_GAUSS_DIAG if diag else _lib.SOL_ROUTE_GAUSS)
    route = _lib.sol_attn_route(rule, float(tau) if beta is None else 0.0, 0.0 if beta is None else float(beta),
                                0 if sinks is None else int(sinks[0]), 0 if sinks is None else int(sinks[1]))
    rc = lib().sol_attn_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, d, 64, 64,
                                        ctypes.byref(route), ctypes.c_uint(flags), _ptr(stats),
                                        _stream(q.device), _ptr(bitmap))
    check(rc, "sol_attn_forward_noalloc")
    return out


def unpack_bitmap(words: torch.Tensor, Nk: int):
    """[..., nwords] int32 words -> [..., Nk] bool numpy array (host)."""
    import numpy as np

    w = words.detach().cpu().numpy().view(np.uint32)
    bits = (w[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1
    return bits.reshape(*w.shape[:-1], -1)[..., :Nk].astype(bool)


class MaskBuilder:
    """Routing alone, for one [B, H, N, d] shape: the kept-block bitmap from
    on-chip threshold routing, or from the top-k / top-p routers that write
    the full proxy map first. ``kpool`` is sol_attn_pool() of k."""

    def __init__(self, B: int, H: int, N: int, d: int, device="cuda", Bq: int = 64, Bk: int = 64):
        self.B, self.H, self.N, self.d, self.Bq, self.Bk = B, H, N, d, Bq, Bk
        self.device = _device(device)
        nbytes = int(lib().sol_attn_mask_workspace_bytes(B, H, N, d, Bq, Bk))
        if nbytes == 0:
            check(_lib.SOL_EUNSUPPORTED, "sol_attn_mask_workspace_bytes")
        self.workspace = torch.empty(-(-nbytes // 8), dtype=torch.int64, device=self.device)
        self.bitmap = torch.zeros(bitmap_shape(B, H, N, Bq, Bk), dtype=torch.int32, device=self.device)

    def _common(self, q, kpool):
        _check_qkv("q", q, (self.B, self.H, self.N, self.d))
        _check_f32("kpool", kpool, pooled_shape(self.B, self.H, self.N, self.d, self.Bk), self.device)
        return (_ptr(q), _ptr(kpool), self.B, self.H, self.N, self.d, self.Bq, self.Bk)

    def threshold(self, q, kpool, tau: float = 0.0, sinks: Optional[Tuple[int, int]] = None) -> torch.Tensor:
        """The forward's own routing (row-max rule, optional sinks), bitmap only."""
        route = _lib.sol_attn_route(_lib.SOL_ROUTE_ROWMAX, float(tau), 0.0,
                                    0 if sinks is None else int(sinks[0]), 0 if sinks is None else int(sinks[1]))
        rc = lib().sol_attn_mask_threshold(*self._common(q, kpool), ctypes.byref(route), _ptr(self.bitmap),
                                           _ptr(self.workspace), self.workspace.numel() * 8, _stream(self.device))
        check(rc, "sol_attn_mask_threshold")
        return self.bitmap

    def topk(self, q, kpool, k: int) -> torch.Tensor:
        rc = lib().sol_attn_mask_topk(*self._common(q, kpool), int(k), _ptr(self.bitmap), _ptr(self.workspace),
                                      self.workspace.numel() * 8, _stream(self.device))
        check(rc, "sol_attn_mask_topk")
        return self.bitmap

    def topp(self, q, kpool, p: float) -> torch.Tensor:
        rc = lib().sol_attn_mask_topp(*self._common(q, kpool), ctypes.c_float(float(p)), _ptr(self.bitmap),
                                      _ptr(self.workspace), self.workspace.numel() * 8, _stream(self.device))
        check(rc, "sol_attn_mask_topp")
        return self.bitmap
