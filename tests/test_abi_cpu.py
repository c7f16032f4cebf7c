"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects every bad argument on the host before launching anything.

Every call below is invalid on purpose; pointer values are fake and are never
dereferenced because validation fails first.
"""
import ctypes
import math
import os
import re

import pytest

import block_sparse_attention_14_amd as sa
from block_sparse_attention_14_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "sol_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(sa.LIB_PATH), reason="libsolattn.so not built")

P = 0x10000  # fake, 16-byte aligned, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sol_attn_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    L = sa.lib()
    for n in names:
        assert getattr(L, n) is not None


def test_strerror():
    for code in (0, -1, -2, -3, -4, -5):
        assert sa.strerror(code) and sa.strerror(code) != sa.strerror(-99)


def test_workspace_bytes():
    L = sa.lib()
    assert L.sol_attn_workspace_bytes(1, 12, 32760, 128, 64, 64) >= 8
    assert L.sol_attn_workspace_bytes(1, 12, 32760, 96, 64, 64) == 0
    assert L.sol_attn_workspace_bytes(1, 12, 32760, 128, 32, 64) == 0
    assert L.sol_attn_workspace_bytes(0, 12, 32760, 128, 64, 64) == 0
    assert L.sol_attn_workspace_bytes(1, 1, sa.SOL_ATTN_MAX_N + 1, 128, 64, 64) == 0


def fwd(**over):
    a = dict(q=P, k=P, v=P, out=P, B=1, H=2, N=1000, d=128, Bq=64, Bk=64, tau=2.0, flags=0, stats=None,
             kpool=P, vmean=P, ws=P, ws_bytes=64, stream=None)
    a.update(over)
    return sa.lib().sol_attn_forward(a["q"], a["k"], a["v"], a["out"], a["B"], a["H"], a["N"], a["d"],
                                     a["Bq"], a["Bk"], ctypes.c_float(a["tau"]), ctypes.c_uint(a["flags"]),
                                     a["stats"], a["kpool"], a["vmean"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(q=None), sa.SOL_EINVAL),
    (dict(k=None), sa.SOL_EINVAL),
    (dict(v=None), sa.SOL_EINVAL),
    (dict(out=None), sa.SOL_EINVAL),
    (dict(kpool=None), sa.SOL_EINVAL),
    (dict(vmean=None), sa.SOL_EINVAL),
    (dict(ws=None), sa.SOL_EINVAL),
    (dict(q=P + 2), sa.SOL_EINVAL),
    (dict(out=P + 4), sa.SOL_EINVAL),
    (dict(ws=P + 4), sa.SOL_EINVAL),
    (dict(ws=P + 128), sa.SOL_EINVAL),
    (dict(flags=sa.SOL_F_PLANNED), sa.SOL_EINVAL),
    (dict(stats=P + 4), sa.SOL_EINVAL),
    (dict(B=0), sa.SOL_EINVAL),
    (dict(H=-1), sa.SOL_EINVAL),
    (dict(N=0), sa.SOL_EINVAL),
    (dict(d=0), sa.SOL_EINVAL),
    (dict(tau=-1e-6), sa.SOL_EINVAL),
    (dict(tau=float("nan")), sa.SOL_EINVAL),
    (dict(tau=-math.inf), sa.SOL_EINVAL),
    (dict(flags=1 << 7), sa.SOL_EINVAL),
    (dict(flags=sa.SOL_F_EXACT_ONLY | sa.SOL_F_ROW_CORRECTION), sa.SOL_EINVAL),
    (dict(d=96), sa.SOL_EUNSUPPORTED),
    (dict(d=256), sa.SOL_EUNSUPPORTED),
    (dict(Bq=32), sa.SOL_EUNSUPPORTED),
    (dict(Bk=128), sa.SOL_EUNSUPPORTED),
    (dict(N=sa.SOL_ATTN_MAX_N + 1), sa.SOL_EUNSUPPORTED),
    (dict(ws_bytes=4), sa.SOL_EWORKSPACE),
])
def test_forward_rejects_before_launch(over, code):
    assert fwd(**over) == code


@pytest.mark.parametrize("args,code", [
    ((None, P, 1, 2, 1000, 128, 64, 64, 2.0, P, 1 << 30, None), sa.SOL_EINVAL),
    ((P, None, 1, 2, 1000, 128, 64, 64, 2.0, P, 1 << 30, None), sa.SOL_EINVAL),
    ((P, P, 1, 2, 1000, 128, 64, 64, 2.0, None, 1 << 30, None), sa.SOL_EINVAL),
    ((P, P, 1, 2, 1000, 128, 64, 64, 2.0, P + 64, 1 << 30, None), sa.SOL_EINVAL),
    ((P, P, 1, 2, 1000, 128, 64, 64, -1.0, P, 1 << 30, None), sa.SOL_EINVAL),
    ((P, P, 1, 2, 1000, 128, 64, 64, float("nan"), P, 1 << 30, None), sa.SOL_EINVAL),
    ((P, P, 0, 2, 1000, 128, 64, 64, 2.0, P, 1 << 30, None), sa.SOL_EINVAL),
    ((P, P, 1, 2, 1000, 96, 64, 64, 2.0, P, 1 << 30, None), sa.SOL_EUNSUPPORTED),
    ((P, P, 1, 2, 1000, 128, 64, 32, 2.0, P, 1 << 30, None), sa.SOL_EUNSUPPORTED),
    ((P, P, 1, 2, 1000, 128, 64, 64, 2.0, P, 64, None), sa.SOL_EWORKSPACE),
])
def test_plan_rejects_before_launch(args, code):
    a = list(args)
    a[8] = ctypes.c_float(a[8])
    assert sa.lib().sol_attn_plan(*a) == code


@pytest.mark.parametrize("args,code", [
    ((None, P, P, 1, 2, 1000, 128, 64, 64, 0, P, 1 << 30, None), sa.SOL_EINVAL),
    ((P, None, P, 1, 2, 1000, 128, 64, 64, 0, P, 1 << 30, None), sa.SOL_EINVAL),
    ((P, P, None, 1, 2, 1000, 128, 64, 64, 0, P, 1 << 30, None), sa.SOL_EINVAL),
    ((P, P, P, 1, 2, 1000, 128, 64, 64, 0, None, 1 << 30, None), sa.SOL_EINVAL),
    ((P, P, P + 4, 1, 2, 1000, 128, 64, 64, 0, P, 1 << 30, None), sa.SOL_EINVAL),
    ((P, P, P, 1, 2, 1000, 128, 64, 64, 0, P + 64, 1 << 30, None), sa.SOL_EINVAL),
    ((P, P, P, 1, 2, 1000, 128, 64, 64, sa.SOL_F_POOLED, P, 1 << 30, None), sa.SOL_EINVAL),
    ((P, P, P, 0, 2, 1000, 128, 64, 64, 0, P, 1 << 30, None), sa.SOL_EINVAL),
    ((P, P, P, 1, 2, 1000, 96, 64, 64, 0, P, 1 << 30, None), sa.SOL_EUNSUPPORTED),
    ((P, P, P, 1, 2, 1000, 128, 64, 64, 0, P, 64, None), sa.SOL_EWORKSPACE),
])
def test_prepare_rejects_before_launch(args, code):
    a = list(args)
    a[9] = ctypes.c_uint(a[9])
    assert sa.lib().sol_attn_prepare(*a) == code


def test_prepared_forward_needs_pooled_inputs():
    # SOL_F_PREPARED reads the caller's pooled tensors' planes: only with SOL_F_POOLED
    assert fwd(flags=sa.SOL_F_PREPARED) == sa.SOL_EINVAL
    assert fwd(flags=sa.SOL_F_PREPARED | sa.SOL_F_PLANNED) == sa.SOL_EINVAL


def test_debug_requires_bitmap():
    L = sa.lib()
    rc = L.sol_attn_forward_debug(P, P, P, P, 1, 2, 1000, 128, 64, 64, ctypes.c_float(2.0), ctypes.c_uint(0),
                                  None, P, P, P, 64, None, None)
    assert rc == sa.SOL_EINVAL
    rc = L.sol_attn_forward_debug(P, P, P, P, 1, 2, 1000, 128, 64, 64, ctypes.c_float(2.0), ctypes.c_uint(0),
                                  None, P, P, P, 64, None, P + 2)
    assert rc == sa.SOL_EINVAL


@pytest.mark.parametrize("args,code", [
    ((None, P, P, P, 1, 2, 100, 128, 64, None), sa.SOL_EINVAL),
    ((P, P, None, P, 1, 2, 100, 128, 64, None), sa.SOL_EINVAL),
    ((P, P + 8, P, P, 1, 2, 100, 128, 64, None), sa.SOL_EINVAL),
    ((P, P, P, P, 1, 2, 0, 128, 64, None), sa.SOL_EINVAL),
    ((P, P, P, P, 1, 2, 100, 80, 64, None), sa.SOL_EUNSUPPORTED),
    ((P, P, P, P, 1, 2, 100, 128, 16, None), sa.SOL_EUNSUPPORTED),
])
def test_pool_rejects_before_launch(args, code):
    assert sa.lib().sol_attn_pool(*args) == code


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _lib.lib()


def fwd_ex(route, bitmap=None, **over):
    a = dict(q=P, k=P, v=P, out=P, B=1, H=2, N=1000, d=128, Bq=64, Bk=64, flags=0, stats=None,
             kpool=P, vmean=P, ws=P, ws_bytes=64, stream=None)
    a.update(over)
    rp = None if route is None else ctypes.byref(_lib.sol_attn_route(*route))
    return sa.lib().sol_attn_forward_ex(a["q"], a["k"], a["v"], a["out"], a["B"], a["H"], a["N"], a["d"],
                                        a["Bq"], a["Bk"], rp, ctypes.c_uint(a["flags"]), a["stats"], a["kpool"],
                                        a["vmean"], a["ws"], a["ws_bytes"], a["stream"], bitmap)


@pytest.mark.parametrize("route,bitmap,code", [
    (None, None, sa.SOL_EINVAL),
    ((7, 1.0, 0.0, 0, 0), None, sa.SOL_EINVAL),                       # unknown rule
    ((0, -1.0, 0.0, 0, 0), None, sa.SOL_EINVAL),                      # negative tau
    ((0, math.nan, 0.0, 0, 0), None, sa.SOL_EINVAL),
    ((1, 0.0, math.inf, 0, 0), None, sa.SOL_EINVAL),                  # beta not finite
    ((1, 0.0, math.nan, 0, 0), None, sa.SOL_EINVAL),
    ((0, 1.0, 0.0, 0, -1), None, sa.SOL_EINVAL),                      # negative sink count
    ((0, 1.0, 0.0, -1, 1), None, sa.SOL_EINVAL),                      # sink range before 0
    ((0, 1.0, 0.0, 15, 2), None, sa.SOL_EINVAL),                      # past Nk = 16
    ((0, 1.0, 0.0, 0, 0), P + 2, sa.SOL_EINVAL),                      # misaligned bitmap
    ((1, 0.0, 1.0, 15, 1), None, sa.SOL_EWORKSPACE),                  # valid route, small workspace
    ((0, math.inf, 0.0, 0, 16), None, sa.SOL_EWORKSPACE),
])
def test_forward_ex_rejects_before_launch(route, bitmap, code):
    assert fwd_ex(route, bitmap) == code


def test_mask_workspace_bytes():
    L = sa.lib()
    n = L.sol_attn_mask_workspace_bytes(1, 12, 32760, 128, 64, 64)
    assert n >= 12 * 512 * 512 * 4 + 12 * 512 * 128 * 4
    assert L.sol_attn_mask_workspace_bytes(1, 12, 32760, 96, 64, 64) == 0
    assert L.sol_attn_mask_workspace_bytes(1, 70000, 64, 128, 64, 64) == 0  # B * H beyond one grid row per head


@pytest.mark.parametrize("args,code", [
    ((None, P, 1, 2, 1000, 128, 64, 64), sa.SOL_EINVAL),
    ((P, None, 1, 2, 1000, 128, 64, 64), sa.SOL_EINVAL),
    ((P + 2, P, 1, 2, 1000, 128, 64, 64), sa.SOL_EINVAL),
    ((P, P, 0, 2, 1000, 128, 64, 64), sa.SOL_EINVAL),
    ((P, P, 1, 2, 1000, 96, 64, 64), sa.SOL_EUNSUPPORTED),
    ((P, P, 1, 70000, 64, 128, 64, 64), sa.SOL_EUNSUPPORTED),
])
def test_mask_builders_reject_before_launch(args, code):
    L = sa.lib()
    route = ctypes.byref(_lib.sol_attn_route(0, 2.0, 0.0, 0, 0))
    assert L.sol_attn_mask_threshold(*args, route, P, P, 1 << 40, None) == code
    assert L.sol_attn_mask_topk(*args, 4, P, P, 1 << 40, None) == code
    assert L.sol_attn_mask_topp(*args, ctypes.c_float(0.9), P, P, 1 << 40, None) == code


def test_mask_builders_reject_bad_route_bitmap_workspace():
    L = sa.lib()
    a = (P, P, 1, 2, 1000, 128, 64, 64)
    good = ctypes.byref(_lib.sol_attn_route(0, 2.0, 0.0, 0, 0))
    assert L.sol_attn_mask_threshold(*a, None, P, P, 1 << 40, None) == sa.SOL_EINVAL
    assert L.sol_attn_mask_threshold(*a, ctypes.byref(_lib.sol_attn_route(1, 0.0, math.nan, 0, 0)), P, P, 1 << 40,
                                     None) == sa.SOL_EINVAL
    assert L.sol_attn_mask_threshold(*a, good, None, P, 1 << 40, None) == sa.SOL_EINVAL
    assert L.sol_attn_mask_threshold(*a, good, P + 2, P, 1 << 40, None) == sa.SOL_EINVAL
    assert L.sol_attn_mask_threshold(*a, good, P, None, 1 << 40, None) == sa.SOL_EINVAL
    assert L.sol_attn_mask_threshold(*a, good, P, P + 64, 1 << 40, None) == sa.SOL_EINVAL
    assert L.sol_attn_mask_threshold(*a, good, P, P, 64, None) == sa.SOL_EWORKSPACE
    # the Gaussian rules are the forward's only (statistics in its workspace)
    assert L.sol_attn_mask_threshold(*a, ctypes.byref(_lib.sol_attn_route(1, 0.0, 1.0, 0, 0)), P, P, 1 << 40,
                                     None) == sa.SOL_EUNSUPPORTED
    assert L.sol_attn_mask_topk(*a, 4, P, None, 1 << 40, None) == sa.SOL_EINVAL
    assert L.sol_attn_mask_topk(*a, 4, P, P + 64, 1 << 40, None) == sa.SOL_EINVAL
    assert L.sol_attn_mask_topk(*a, 4, P, P, 64, None) == sa.SOL_EWORKSPACE
    assert L.sol_attn_mask_topp(*a, ctypes.c_float(math.nan), P, P, 1 << 40, None) == sa.SOL_EINVAL


@pytest.mark.parametrize("rule", [1, 2])
def test_exact_only_under_a_gaussian_rule_needs_sinks(rule):
    """A Gaussian threshold above a query block's best proxy keeps nothing;
    without the correction such a block's rows would have no term at all, so
    exact-only is refused there unless sink blocks guarantee a kept block."""
    EO = sa.SOL_F_EXACT_ONLY
    assert fwd_ex((rule, 0.0, 50.0, 0, 0), flags=EO) == sa.SOL_EINVAL
    assert fwd_ex((rule, 0.0, 0.0, 0, 0), flags=EO) == sa.SOL_EINVAL
    # with a sink range (or the correction) the same route passes validation
    assert fwd_ex((rule, 0.0, 50.0, 3, 1), flags=EO) == sa.SOL_EWORKSPACE
    assert fwd_ex((rule, 0.0, 50.0, 0, 0)) == sa.SOL_EWORKSPACE
    # the row-max rule always keeps its best block
    assert fwd_ex((0, 0.0, 0.0, 0, 0), flags=EO) == sa.SOL_EWORKSPACE


def fwd_noalloc(route=(0, 2.0, 0.0, 0, 0), bitmap=None, **over):
    a = dict(q=P, k=P, v=P, out=P, B=1, H=2, N=1000, d=128, Bq=64, Bk=64, flags=0, stats=None, stream=None)
    a.update(over)
    rp = None if route is None else ctypes.byref(_lib.sol_attn_route(*route))
    return sa.lib().sol_attn_forward_noalloc(a["q"], a["k"], a["v"], a["out"], a["B"], a["H"], a["N"], a["d"],
                                             a["Bq"], a["Bk"], rp, ctypes.c_uint(a["flags"]), a["stats"],
                                             a["stream"], bitmap)


@pytest.mark.parametrize("route,over,code", [
    (None, {}, sa.SOL_EINVAL),
    ((0, -1.0, 0.0, 0, 0), {}, sa.SOL_EINVAL),
    ((0, 2.0, 0.0, 0, 0), dict(q=None), sa.SOL_EINVAL),
    ((0, 2.0, 0.0, 0, 0), dict(out=P + 4), sa.SOL_EINVAL),
    ((0, 2.0, 0.0, 0, 0), dict(flags=sa.SOL_F_POOLED), sa.SOL_EINVAL),
    ((0, 2.0, 0.0, 0, 0), dict(flags=sa.SOL_F_POOLED | sa.SOL_F_PLANNED), sa.SOL_EINVAL),
    ((0, 2.0, 0.0, 0, 0), dict(flags=sa.SOL_F_POOLED | sa.SOL_F_PREPARED), sa.SOL_EINVAL),
    ((1, 0.0, 1.0, 0, 0), dict(flags=sa.SOL_F_EXACT_ONLY), sa.SOL_EINVAL),
    ((0, 2.0, 0.0, 0, 0), dict(d=96), sa.SOL_EUNSUPPORTED),
    # 64 heads of 118800 tokens need about 190 MiB of pooled buffers: beyond the array
    ((0, 2.0, 0.0, 0, 0), dict(H=64, N=118800), sa.SOL_ESCRATCH),
    ((0, 2.0, 0.0, 0, 0), dict(H=1, N=sa.SOL_ATTN_MAX_N, B=40), sa.SOL_ESCRATCH),
])
def test_noalloc_rejects_before_launch(route, over, code):
    assert fwd_noalloc(route, **over) == code


def test_noalloc_scratch_limit():
    """The array's size is the header's constant; the 119K-token layer (24
    heads, d = 128) fits in it in every mode."""
    assert sa.SOL_ATTN_SCRATCH_BYTES == 128 << 20
    text = open(HEADER).read()
    assert "#define SOL_ATTN_SCRATCH_BYTES (128u << 20)" in text
    L = sa.lib()
    ws = L.sol_attn_workspace_bytes(1, 24, 118800, 128, 64, 64)
    pooled = -(-(24 * 1857 * 128 * 4) // 256) * 256
    assert ws + 2 * pooled <= sa.SOL_ATTN_SCRATCH_BYTES


@pytest.mark.parametrize("over,code", [
    (dict(flags=sa.SOL_F_GROUP2), sa.SOL_EWORKSPACE),       # valid: the small workspace fails next
    (dict(flags=sa.SOL_F_GROUP4), sa.SOL_EWORKSPACE),
    (dict(flags=sa.SOL_F_GROUP8), sa.SOL_EWORKSPACE),
    (dict(flags=sa.SOL_F_GROUP16), sa.SOL_EWORKSPACE),
    (dict(flags=sa.SOL_F_GROUP6), sa.SOL_EWORKSPACE),
    (dict(flags=sa.SOL_F_GROUP6, N=2048 * 64 + 1), sa.SOL_EWORKSPACE),
    (dict(flags=sa.SOL_F_GROUP6 | sa.SOL_F_GROUP16), sa.SOL_EINVAL),
    (dict(flags=sa.SOL_F_GROUP6 | sa.SOL_F_GROUP2), sa.SOL_EINVAL),
    # eight or sixteen query blocks per item only up to 2048 key blocks
    (dict(flags=sa.SOL_F_GROUP8, N=2048 * 64 + 1), sa.SOL_EUNSUPPORTED),
    (dict(flags=sa.SOL_F_GROUP16, N=2048 * 64 + 1), sa.SOL_EUNSUPPORTED),
    (dict(flags=sa.SOL_F_GROUP16, N=2048 * 64), sa.SOL_EWORKSPACE),
    # one size at most
    (dict(flags=sa.SOL_F_GROUP16 | sa.SOL_F_GROUP4), sa.SOL_EINVAL),
    (dict(flags=sa.SOL_F_GROUP4, N=2048 * 64 + 1), sa.SOL_EWORKSPACE),
    # a plan orders the items of the automatic group size
    (dict(flags=sa.SOL_F_GROUP2 | sa.SOL_F_POOLED | sa.SOL_F_PLANNED), sa.SOL_EINVAL),
    (dict(flags=sa.SOL_F_GROUP16 | sa.SOL_F_POOLED | sa.SOL_F_PLANNED), sa.SOL_EINVAL),
    (dict(flags=1 << 10), sa.SOL_EINVAL),                    # unknown bit
])
def test_group_field_of_the_flags(over, code):
    assert fwd(**over) == code


def test_forward_ex_accepts_diag_rule_arguments():
    # a valid diagonal-estimator route passes validation (the tiny workspace fails next)
    assert fwd_ex((2, 0.0, 1.0, 0, 0)) == sa.SOL_EWORKSPACE
    assert fwd_ex((2, 0.0, math.inf, 0, 0)) == sa.SOL_EINVAL
    assert fwd_ex((3, 0.0, 1.0, 0, 0)) == sa.SOL_EINVAL


def test_header_is_plain_c():
    """The header compiles as strict C99 and as C++ (no torch or HIP types needed)."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    inc = os.path.dirname(HEADER)
    for lang, std in (("c", "-std=c99"), ("c++", "-std=c++17")):
        r = subprocess.run([gcc, "-x", lang, std, "-pedantic", "-Wall", "-Werror", "-fsyntax-only", "-I", inc, "-"],
                           input='#include "sol_attn.h"\n', text=True, capture_output=True)
        assert r.returncode == 0, r.stderr


def test_c_example_links_against_the_library():
    """The C example built beside the library resolves libsolattn through its run path."""
    import subprocess

    exe = os.path.join(os.path.dirname(sa.LIB_PATH), "sol_attn_example")
    if not os.path.exists(exe):
        pytest.skip("C example not built")
    r = subprocess.run(["ldd", exe], text=True, capture_output=True)
    assert r.returncode == 0, r.stderr
    assert "not found" not in r.stdout, r.stdout
    line = [ln for ln in r.stdout.splitlines() if "libsolattn.so" in ln]
    assert line and os.path.realpath(sa.LIB_PATH) in os.path.realpath(line[0].split("=>")[1].split()[0])
