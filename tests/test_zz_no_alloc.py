"""sol_attn_forward_noalloc (the forward over the library's static device
scratch array) against sol_attn_forward_ex (the same forward over the
caller's buffers), through the C ABI, on consecutive calls of different sizes.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_14_amd as sa
from workloads import Workload, get_workload, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sa.lib()


def _tensors(wl):
    x = make_inputs(wl)
    return tuple(torch.from_numpy(x[n].view(np.int16)).cuda().view(torch.bfloat16) for n in "qkv")


def _reference(q, k, v, tau, **kw):
    B, H, N, d = q.shape
    r = sa.SolAttention(B, H, N, d, q.device)
    bm = torch.zeros(sa.bitmap_shape(B, H, N), dtype=torch.int32, device=q.device)
    out = r(q, k, v, tau, bitmap=bm, **kw)
    torch.cuda.synchronize()
    return out.clone(), bm.clone(), r.read_stats()


def _noalloc(q, k, v, tau, **kw):
    B, H, N, d = q.shape
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device)
    bm = torch.full(sa.bitmap_shape(B, H, N), -1, dtype=torch.int32, device=q.device)
    st = sa.new_stats(q.device)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated(q.device)
    sa.forward_noalloc(q, k, v, out, tau, stats=st, bitmap=bm, **kw)
    after = torch.cuda.memory_allocated(q.device)
    torch.cuda.synchronize()
    assert after == before  # nothing allocated on the way to the library
    return out, bm, sa.read_stats(st)


def _same(a, b, where):
    out_a, bm_a, st_a = a
    out_b, bm_b, st_b = b
    assert torch.equal(out_a.view(torch.int32), out_b.view(torch.int32)), f"{where}: outputs differ"
    assert torch.equal(bm_a, bm_b), f"{where}: bitmaps differ"
    assert st_a == st_b, f"{where}: stats differ"
    print(f"[no-alloc] {where}: identical to sol_attn_forward_ex, kept {st_a['kept_blocks']}/{st_a['total_blocks']}",
          flush=True)


def test_noalloc_matches_forward_on_consecutive_calls():
    """A 4K image layer at tau = 8 (planned by default), then a smaller ragged
    layer at tau = 2 (the array now holds the first call's workspace and
    pooled buffers), then the Gaussian rule with sinks on the small layer,
    then the large layer again: each equals the caller-buffer forward bit for
    bit, stats and routing included."""
    big = _tensors(get_workload("image_dit_4k"))
    small = _tensors(Workload(name="small", B=1, H=3, grid=(1, 1, 1000), d=64, dtype="bf16", taus=(), seed=41))
    _same(_noalloc(*big, 8.0), _reference(*big, 8.0), "image_dit_4k tau=8")
    _same(_noalloc(*small, 2.0), _reference(*small, 2.0), "N=1000 d=64 tau=2")
    _same(_noalloc(*small, 0.0, beta=0.5, sinks=(2, 1)), _reference(*small, 0.0, beta=0.5, sinks=(2, 1)),
          "N=1000 d=64 gauss beta=0.5 sinks")
    _same(_noalloc(*big, math.inf), _reference(*big, math.inf), "image_dit_4k tau=inf")


def test_noalloc_per_row_correction_and_bf16_out():
    x = _tensors(Workload(name="rc", B=1, H=2, grid=(1, 1, 1300), d=128, dtype="bf16", taus=(), seed=43))
    _same(_noalloc(*x, 1.0, flags=sa.SOL_F_ROW_CORRECTION), _reference(*x, 1.0, flags=sa.SOL_F_ROW_CORRECTION),
          "N=1300 d=128 per-row correction")
    q = x[0]
    ref = sa.SolAttention(*q.shape, q.device)(*x, 1.0, out_dtype=torch.bfloat16)
    out16 = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    sa.forward_noalloc(*x, out16, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(out16.view(torch.int16), ref.view(torch.int16))


def test_noalloc_rejects_before_launch():
    x = _tensors(Workload(name="rej", B=1, H=1, grid=(1, 1, 200), d=128, dtype="bf16", taus=(), seed=45))
    out = torch.empty(x[0].shape, dtype=torch.float32, device=x[0].device)
    for kw in (dict(flags=sa.SOL_F_POOLED), dict(flags=sa.SOL_F_POOLED | sa.SOL_F_PLANNED), dict(tau=-1.0)):
        with pytest.raises(sa.SolAttnError) as e:
            sa.forward_noalloc(*x, out, **({"tau": 2.0} | kw))
        assert e.value.code == sa.SOL_EINVAL
