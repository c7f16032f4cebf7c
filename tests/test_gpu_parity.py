"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Bars: routing bitmap exact away from a 1e-3 band around the threshold; output
max-abs error <= 2e-2 with the oracle conditioned on the GPU's routing; stats
equal to what the exported bitmap implies; bitwise-deterministic reruns.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_14_amd as sa
from oracle import attend_head, block_means
from workloads import Workload, bf16_bits_to_f64, get_workload, make_inputs

from parity import check_head, check_stats, run_gpu, sample_blocks, stratified_blocks, to_device_bf16

pytestmark = pytest.mark.gpu

INF = math.inf


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sa.lib()


def _report(name, tag, err):
    print(f"[parity] {name} {tag} max_abs_err={err:.3e}", flush=True)


def _full_parity(wl: Workload, tau, inputs=None, query_blocks_per_head=None, seed=0, beta=None, sinks=None,
                 flags=0, diag=False, stratified=False, whole_heads=(), heads=None, group=0):
    """GPU call through the C ABI, then per head: the bitmap on every query
    block; outputs on every row (default), on `query_blocks_per_head` random
    blocks, or (stratified=True) on the scheduling-stratified sample plus the
    `whole_heads` checked on every row. `heads` limits the checked heads."""
    x = inputs or make_inputs(wl)
    flags |= sa.api.group_flag(group)
    out, keep, stats = run_gpu(x["q"], x["k"], x["v"], tau, beta=beta, sinks=sinks, flags=flags, diag=diag)
    check_stats(stats, keep, wl.N)
    rng = np.random.default_rng(seed)
    strat = stratified_blocks(wl.B, wl.H, wl.Nq, rng) if stratified else None
    worst = 0.0
    tag = f"tau={tau}" if beta is None else f"beta={beta}" + (" diag" if diag else "")
    if sinks is not None:
        tag += f" sinks={sinks}"
    rowc = bool(flags & sa.SOL_F_ROW_CORRECTION)
    if rowc:
        tag += " row-correction"
    if group:
        tag += f" group={group}"
    if flags & sa.SOL_F_EXACT_ONLY:
        tag += " exact-only"
    checked = 0
    for b in range(wl.B):
        for h in range(wl.H):
            if heads is not None and h not in heads:
                continue
            if strat is not None:
                qbs = None if h in whole_heads else strat[(b, h)]
            else:
                qbs = None if query_blocks_per_head is None else sample_blocks(wl.Nq, rng, query_blocks_per_head)
            checked += wl.Nq if qbs is None else len(qbs)
            worst = max(worst, check_head(x["q"][b, h], x["k"][b, h], x["v"][b, h], out[b, h], keep[b, h],
                                          tau, qbs, where=f"{wl.name} b={b} h={h} {tag}", beta=beta, sinks=sinks,
                                          row_correction=rowc, diag=diag,
                                          correction=not (flags & sa.SOL_F_EXACT_ONLY)))
    _report(wl.name, tag + f" query_blocks_checked={checked}", worst)
    return out, keep, stats


# ---------------------------------------------------------------------------
# small shapes: full oracle on every row
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("tau", [0.0, 2.0, 4.0, INF])
def test_tiny_fp32_layer(tau):
    _full_parity(get_workload("tiny_fp32"), tau)


def _custom(N, d, H=3, B=1, seed=77, grid=None):
    return Workload(name=f"custom_N{N}_d{d}", B=B, H=H, grid=grid or (1, 1, N), d=d, dtype="bf16",
                    taus=(), seed=seed)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 40, 63, 64, 65, 130, 1000])
@pytest.mark.parametrize("tau", [0.0, 1.5, INF])
def test_ragged_and_edge_lengths(N, d, tau):
    _full_parity(_custom(N, d, H=2, seed=N + d), tau)


@pytest.mark.parametrize("tau", [2.0, 4.0, 8.0])
def test_image_dit_4k(tau):
    _full_parity(get_workload("image_dit_4k"), tau)


# ---------------------------------------------------------------------------
# the video-sized layers: bitmap on every query block; outputs on every row of
# every head where the oracle runs in seconds (the 32K layers at finite tau),
# else on a sample stratified over the work queues plus whole heads
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def video32k():
    return make_inputs(get_workload("video_dit_32k"))


@pytest.mark.parametrize("tau", [2.0, 4.0, 8.0])
def test_video_dit_32k(video32k, tau):
    """Every row of all 12 heads (tau = 8 is the planned, heaviest-first
    order of the default call)."""
    _full_parity(get_workload("video_dit_32k"), tau, video32k)


def test_video_dit_32k_dense(video32k):
    """tau = +inf (dense: the oracle takes minutes per head): the stratified
    sample, and head 5 on every row."""
    _full_parity(get_workload("video_dit_32k"), INF, video32k, stratified=True, whole_heads=(5,), seed=99)


@pytest.fixture(scope="module")
def imbalance32k():
    return make_inputs(get_workload("video_dit_32k_imbalance"))


@pytest.mark.parametrize("heads", [(0, 1, 2, 3, 4, 5), (6, 7), (8, 9), (10, 11)])
def test_video_dit_32k_imbalance(imbalance32k, heads):
    """Every row of every head, in four groups of heads (the diffuse heads
    6-11 keep every block, so each is a dense head for the oracle)."""
    wl = get_workload("video_dit_32k_imbalance")
    out, keep, stats = _full_parity(wl, 8.0, imbalance32k, heads=heads)
    per_q = keep.sum(axis=-1)
    # sink heads route almost nothing, diffuse heads route almost everything
    assert per_q[0, 6:].mean() > 0.5 * wl.Nk
    assert per_q[0, :2].mean() < 0.05 * wl.Nk


@pytest.fixture(scope="module")
def mild32k():
    return make_inputs(get_workload("video_dit_32k_mild"))


@pytest.mark.parametrize("tau", [1.0, 2.0])
def test_video_dit_32k_mild(mild32k, tau):
    """The milder-locality layer with smooth values: every row of all 12
    heads, block-level correction, and the per-row correction's stratified
    sample with head 7 on every row."""
    wl = get_workload("video_dit_32k_mild")
    _full_parity(wl, tau, mild32k)
    _full_parity(wl, tau, mild32k, flags=RC, stratified=True, whole_heads=(7,), seed=int(tau) + 40)


def test_video_dit_32k_mild_tau4(mild32k):
    """tau = 4 keeps about a third of the blocks here: the stratified sample and
    head 2 on every row."""
    _full_parity(get_workload("video_dit_32k_mild"), 4.0, mild32k, stratified=True, whole_heads=(2,), seed=44)


@pytest.mark.parametrize("tau", [1.0, 2.0])
def test_correction_ablation_on_the_gpu(mild32k, tau):
    """§4 "Ablations" on the GPU: against this kernel's dense output (tau =
    +inf) on the mild layer, per-row correction < block-level correction <
    exact-only attention over the same kept blocks, in relative L2 error over
    all 12 heads (the oracle pins the same order on a reduced layer)."""
    wl = get_workload("video_dit_32k_mild")
    q, k, v = (to_device_bf16(mild32k[n]) for n in "qkv")
    r = sa.SolAttention(wl.B, wl.H, wl.N, wl.d)
    dense = r(q, k, v, INF).double()

    def err(flags):
        o = r(q, k, v, tau, flags=flags).double()
        return float((o - dense).norm() / dense.norm())

    blk, row, exact = err(0), err(RC), err(sa.SOL_F_EXACT_ONLY)
    print(f"[ablation] video_dit_32k_mild tau={tau}: row {row:.4f} block {blk:.4f} exact-only {exact:.4f}", flush=True)
    assert row < blk < exact, (row, blk, exact)
    assert blk < 0.85 * exact, (blk, exact)


@pytest.fixture(scope="module")
def video119k():
    return make_inputs(get_workload("video_dit_119k"))


@pytest.mark.parametrize("tau,whole", [(2.0, 3), (4.0, 11), (8.0, 23)])
def test_video_dit_119k(video119k, tau, whole):
    """The stratified sample over the work queues and one whole head per tau
    (the library routes eight query blocks per work item here)."""
    _full_parity(get_workload("video_dit_119k"), tau, video119k, stratified=True, whole_heads=(whole,),
                 seed=int(tau))


def test_video_dit_119k_router_and_group_sizes(video119k):
    """On the 119K layer: the library's own choice is sixteen query blocks per
    item; the threshold router (the fused kernel stopped after routing, four
    blocks per item) exports the bitmap of the forward with four blocks per
    item bit for bit; groups of two, four, eight and sixteen query blocks
    route alike away from the tie band (their scores are summed in different
    orders), give outputs within the bar of each other where they route
    alike, and match the oracle on their own routing where they do not."""
    from parity import BITMAP_TIE, oracle_route

    wl = get_workload("video_dit_119k")
    q, k, v = (to_device_bf16(video119k[n]) for n in "qkv")
    r = sa.SolAttention(wl.B, wl.H, wl.N, wl.d)
    tau = 4.0
    outs, bms = {}, {}
    for g in (0, 2, 4, 8, 16):
        bm = torch.zeros(sa.bitmap_shape(wl.B, wl.H, wl.N), dtype=torch.int32, device=q.device)
        outs[g] = r(q, k, v, tau, bitmap=bm, group=g).clone()
        bms[g] = bm
    torch.cuda.synchronize()
    assert torch.equal(bms[0], bms[16]) and torch.equal(outs[0].view(torch.int32), outs[16].view(torch.int32))
    mb = sa.MaskBuilder(wl.B, wl.H, wl.N, wl.d)
    assert torch.equal(mb.threshold(q, r.kpool, tau=tau), bms[4])
    keep8 = sa.unpack_bitmap(bms[16], wl.Nk)[0]
    out8 = outs[16].cpu().numpy()[0]
    for g in (2, 4, 8):
        keep = sa.unpack_bitmap(bms[g], wl.Nk)[0]
        out = outs[g].cpu().numpy()[0]
        rows_differ = (keep != keep8).any(axis=-1)  # [H, Nq]
        same = np.repeat(~rows_differ, 64, axis=1)[:, :wl.N]
        err = np.abs(out - out8).max(axis=-1)[same].max()
        print(f"[parity] video_dit_119k group {g} vs 16: {int(rows_differ.sum())} query blocks route differently, "
              f"max abs diff elsewhere {err:.3e}", flush=True)
        assert err <= 2e-2
        for h, i in np.argwhere(rows_differ)[:8]:
            qh, kh, vh = (bf16_bits_to_f64(video119k[n][0, h]) for n in "qkv")
            sc, theta, _, _ = oracle_route(qh, kh, tau)
            flip = keep[h, i] != keep8[h, i]
            assert (np.abs(sc[i, flip] - theta[i]) <= BITMAP_TIE).all(), "a decision differs away from the threshold"
            for kk, oo in ((keep[h], out[h]), (keep8[h], out8[h])):
                ref = attend_head(qh, kh, vh, 64, 64, tau, keep_override=kk, query_blocks=[i])["out"]
                sl = slice(64 * i, min(wl.N, 64 * i + 64))
                assert np.abs(oo[sl] - ref[sl]).max() <= 2e-2


@pytest.mark.parametrize("group", [2, 4, 6, 8, 16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [65, 1000, 4000])
@pytest.mark.parametrize("tau", [0.0, 2.0, INF])
def test_group_sizes(group, d, N, tau):
    """Every group size on ragged heads: 2, 16 and 63 query blocks, so that
    groups of four, six, eight and sixteen end partial (63 = 10 x 6 + 3 =
    7 x 8 + 7 = 3 x 16 + 15), on every row."""
    _full_parity(_custom(N, d, H=2, seed=N + d + group), tau, group=group)


@pytest.mark.parametrize("group", [4, 6, 8, 16])
def test_group_sizes_gauss_sinks_and_row_correction(group):
    wl = _custom(4000, 128, H=2, seed=88)
    _full_parity(wl, 0.0, beta=1.0, group=group)
    _full_parity(wl, 0.0, beta=2.0, diag=True, sinks=(5, 3), group=group)
    _full_parity(wl, 1.0, flags=sa.SOL_F_ROW_CORRECTION, group=group)
    _full_parity(wl, 1.0, sinks=(60, 3), flags=sa.SOL_F_EXACT_ONLY, group=group)


@pytest.mark.parametrize("group", [8, 16])
def test_group8_far_maximum_rechecks_early_candidates(group):
    """A long head (1500 key blocks, six routing chunks) whose best blocks are
    sink blocks at the start of the sequence: every group meets its maximum
    in a late chunk, so blocks kept against the running maximum of earlier
    chunks are rechecked and moved to the correction. Every row checked."""
    wl = Workload(name="sink_far_N96000_d64", B=1, H=2, grid=(1, 1, 96000), d=64, dtype="bf16", taus=(), seed=515,
                  locality=(3.0, 3.0), sink_heads=(0, 1), sink_blocks=4)
    for tau in (2.0, 6.0):
        _full_parity(wl, tau, group=group)


def test_row_correction_video_dit_119k(video119k):
    """Per-row correction at the 119K layer's size: every row scored against
    1857 pooled keys in 29 pooled tiles, the last key block ragged (16
    tokens); outputs on sampled query blocks."""
    _full_parity(get_workload("video_dit_119k"), 2.0, video119k, stratified=True, whole_heads=(7,), seed=12,
                 flags=sa.SOL_F_ROW_CORRECTION)


@pytest.mark.parametrize("d,tau", [(128, 2.0), (64, 4.0), (128, INF)])
def test_maximum_length(d, tau):
    """The longest supported head: N = SOL_ATTN_MAX_N - 1 = 262143 tokens on a
    19 x 73 x 189 grid, 4096 key blocks, the last one ragged (63 tokens).
    Bitmap on every query block, outputs on sampled blocks."""
    N = sa.SOL_ATTN_MAX_N - 1
    assert 19 * 73 * 189 == N
    wl = Workload(name=f"max_N{N}_d{d}", B=1, H=1, grid=(19, 73, 189), d=d, dtype="bf16", taus=(), seed=2024 + d)
    assert wl.Nk == 4096
    _full_parity(wl, tau, query_blocks_per_head=3, seed=d)


def test_maximum_length_row_correction():
    """The longest head with the per-row correction: 64 pooled tiles per item,
    the last one holding the ragged 63-token block."""
    N = sa.SOL_ATTN_MAX_N - 1
    wl = Workload(name=f"max_N{N}_d128", B=1, H=1, grid=(19, 73, 189), d=128, dtype="bf16", taus=(), seed=2152)
    _full_parity(wl, 2.0, query_blocks_per_head=3, seed=5, flags=sa.SOL_F_ROW_CORRECTION)


# ---------------------------------------------------------------------------
# behaviour of the boundary
# ---------------------------------------------------------------------------

def test_deterministic_reruns(video32k):
    a, ka, _ = run_gpu(video32k["q"], video32k["k"], video32k["v"], 4.0)
    b, kb, _ = run_gpu(video32k["q"], video32k["k"], video32k["v"], 4.0)
    assert (ka == kb).all()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("d", [64, 128])
def test_pool_pass_matches_block_means(d):
    wl = _custom(1000, d, H=3, B=2, seed=5)
    x = make_inputs(wl)
    k, v = to_device_bf16(x["k"]), to_device_bf16(x["v"])
    kp, vm = sa.pool(k, v)
    torch.cuda.synchronize()
    kp, vm = kp.cpu().numpy(), vm.cpu().numpy()
    for b in range(wl.B):
        for h in range(wl.H):
            ek, _ = block_means(bf16_bits_to_f64(x["k"][b, h]), 64)
            ev, _ = block_means(bf16_bits_to_f64(x["v"][b, h]), 64)
            np.testing.assert_allclose(kp[b, h], ek, rtol=0, atol=2e-6 * max(1.0, np.abs(ek).max()))
            np.testing.assert_allclose(vm[b, h], ev, rtol=0, atol=2e-6 * max(1.0, np.abs(ev).max()))


def test_pooled_flag_and_stream_reuse():
    wl = get_workload("image_dit_4k")
    x = make_inputs(wl, heads=[(0, h) for h in range(wl.H)] + [(1, h) for h in range(wl.H)])
    q, k, v = (to_device_bf16(x[n]) for n in "qkv")
    r = sa.SolAttention(wl.B, wl.H, wl.N, wl.d)
    base = r(q, k, v, 4.0).clone()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        sa.pool(k, v, kpool=r.kpool, vmean=r.vmean)
        again = r(q, k, v, 4.0, flags=sa.SOL_F_POOLED)
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(base.view(torch.int32), again.view(torch.int32))


def test_concurrent_calls_on_two_streams():
    """Two instances (separate workspaces) running at once on two streams give
    the results of sequential calls bit for bit: no state is shared between
    calls beyond the workspace (the fused kernel never waits on other
    workgroups, so the two persistent grids cannot block each other)."""
    wl = get_workload("image_dit_4k")
    x = make_inputs(wl)
    q, k, v = (to_device_bf16(x[n]) for n in "qkv")
    r1 = sa.SolAttention(wl.B, wl.H, wl.N, wl.d)
    r2 = sa.SolAttention(wl.B, wl.H, wl.N, wl.d)
    ref1 = r1(q, k, v, 2.0).clone()
    ref2 = r2(q, k, v, 8.0).clone()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        with torch.cuda.stream(s1):
            o1 = r1(q, k, v, 2.0)
        with torch.cuda.stream(s2):
            o2 = r2(q, k, v, 8.0)
        s1.synchronize()
        s2.synchronize()
        assert torch.equal(o1.view(torch.int32), ref1.view(torch.int32))
        assert torch.equal(o2.view(torch.int32), ref2.view(torch.int32))


@pytest.mark.parametrize("wlname", ["image_dit_4k", "video_dit_32k"])
def test_hip_graph_capture_and_replay(wlname, request):
    """The whole default call (pool pass, planning where it runs, fused
    kernel: kernels only, no memsets or allocations) captured in a graph and
    replayed several times, with eager calls on the same workspace in
    between, gives the eager result bit for bit on every replay."""
    wl = get_workload(wlname)
    x = request.getfixturevalue("video32k") if wlname == "video_dit_32k" else make_inputs(wl)
    q, k, v = (to_device_bf16(x[n]) for n in "qkv")
    r = sa.SolAttention(wl.B, wl.H, wl.N, wl.d)
    tau = 8.0
    ref = r(q, k, v, tau).clone()  # eager (also sets up the library's per-device state)
    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        r(q, k, v, tau, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        r(q, k, v, tau, out=out)
    for _ in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
        eager = r(q, k, v, tau)
        torch.cuda.synchronize()
        assert torch.equal(eager.view(torch.int32), ref.view(torch.int32))


def test_exact_only_ablation():
    wl = _custom(1000, 128, H=2, seed=9)
    x = make_inputs(wl)
    out, keep, _ = run_gpu(x["q"], x["k"], x["v"], 1.0, flags=sa.SOL_F_EXACT_ONLY)
    for h in range(wl.H):
        q, k, v = (bf16_bits_to_f64(x[n][0, h]) for n in "qkv")
        r = attend_head(q, k, v, 64, 64, 1.0, keep_override=keep[0, h], correction=False)
        err = np.abs(out[0, h] - r["out"]).max()
        assert err <= 2e-2, err


@pytest.mark.parametrize("flags,tau", [(0, INF), (0, 0.0), (sa.SOL_F_ROW_CORRECTION, 0.0),
                                       (sa.SOL_F_ROW_CORRECTION, INF), (sa.SOL_F_EXACT_ONLY, 0.0)])
def test_row_far_below_its_block_proxy(flags, tau):
    """A query row anti-aligned with the rest of its block: its exact logits
    lie thousands of units below the block's proxy maximum. With no
    correction mass (every block kept, the per-row mode, exact-only) the
    row's own exact terms must still be normalised on their own maximum, as
    the oracle does, instead of vanishing under the proxy's."""
    from workloads import f32_to_bf16_bits

    N, d = 192, 64
    rng = np.random.default_rng(404)
    one = np.ones(d, np.float32)
    q = (3.0 * one + 0.1 * rng.standard_normal((N, d))).astype(np.float32)
    q[0] = -100.0 * one
    q[70] = -60.0 * one
    k = (3.0 * one + 0.5 * rng.standard_normal((N, d))).astype(np.float32)
    v = rng.standard_normal((N, d)).astype(np.float32)
    qb, kb, vb = (f32_to_bf16_bits(x)[None, None] for x in (q, k, v))
    out, keep, _ = run_gpu(qb, kb, vb, tau, flags=flags)
    assert np.isfinite(out).all()
    qf, kf, vf = (bf16_bits_to_f64(x[0, 0]) for x in (qb, kb, vb))
    r = attend_head(qf, kf, vf, 64, 64, tau, keep_override=keep[0, 0],
                    correction=not (flags & sa.SOL_F_EXACT_ONLY),
                    row_correction=bool(flags & sa.SOL_F_ROW_CORRECTION))
    err = np.abs(out[0, 0] - r["out"]).max()
    _report("anti_aligned_rows", f"flags={flags} tau={tau}", err)
    assert err <= 2e-2


def test_invalid_arguments_raise():
    wl = _custom(100, 128, H=1)
    x = make_inputs(wl)
    q, k, v = (to_device_bf16(x[n]) for n in "qkv")
    r = sa.SolAttention(1, 1, 100, 128)
    with pytest.raises(sa.SolAttnError):
        r(q, k, v, -1.0)
    with pytest.raises(sa.SolAttnError):
        r(q, k, v, float("nan"))


def test_plan_then_planned_forwards_match_one_shot():
    """sol_attn_pool + sol_attn_plan + forward(POOLED|PLANNED), twice, equals
    the one-shot forward bit for bit; stats are right on every call (the
    fused kernel leaves its queue and stat words clean)."""
    wl = get_workload("image_dit_4k")
    x = make_inputs(wl)
    q, k, v = (to_device_bf16(x[n]) for n in "qkv")
    one = sa.SolAttention(wl.B, wl.H, wl.N, wl.d)
    ref = one(q, k, v, 4.0).clone()
    ref_stats = one.read_stats()
    r = sa.SolAttention(wl.B, wl.H, wl.N, wl.d)
    sa.pool(k, v, kpool=r.kpool, vmean=r.vmean)
    r.plan(q, 4.0)
    for _ in range(2):
        out = r(q, k, v, 4.0, flags=sa.SOL_F_POOLED | sa.SOL_F_PLANNED)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
        assert r.read_stats() == ref_stats
    # dense: no order, still one kernel
    dense_ref = one(q, k, v, INF).clone()
    r.plan(q, INF)
    out = r(q, k, v, INF, flags=sa.SOL_F_POOLED | sa.SOL_F_PLANNED)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), dense_ref.view(torch.int32))


def test_prepared_forwards_match_one_shot():
    """sol_attn_pool + sol_attn_prepare (+ sol_attn_plan) + forward with
    SOL_F_PREPARED launches only the fused kernel (and a reset when unplanned)
    and equals the one-shot forward bit for bit, also with the per-row
    correction; stats are right on every call."""
    wl = get_workload("image_dit_4k")
    x = make_inputs(wl)
    q, k, v = (to_device_bf16(x[n]) for n in "qkv")
    one = sa.SolAttention(wl.B, wl.H, wl.N, wl.d)
    r = sa.SolAttention(wl.B, wl.H, wl.N, wl.d)
    sa.pool(k, v, kpool=r.kpool, vmean=r.vmean)
    for extra in (0, sa.SOL_F_ROW_CORRECTION):
        ref = one(q, k, v, 8.0, flags=extra).clone()
        ref_stats = one.read_stats()
        r.prepare(q, flags=extra)
        for planned in (False, True, True):
            flags = sa.SOL_F_POOLED | sa.SOL_F_PREPARED | extra
            if planned:
                r.plan(q, 8.0)
                flags |= sa.SOL_F_PLANNED
            out = r(q, k, v, 8.0, flags=flags)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), (extra, planned)
            assert r.read_stats() == ref_stats
    print(f"[prepared] image_dit_4k tau=8: prepared forwards identical to one-shot, kept {ref_stats['kept_blocks']}",
          flush=True)


def test_plan_for_another_group_size_is_ignored(video119k):
    """On the 119K layer the library routes sixteen query blocks per item at
    tau <= 4 and eight above: a plan made at one tau and followed by a
    planned forward at the other is for another item count, so the fused
    kernel takes the items in sequence and the result equals the unplanned
    forward bit for bit (and the matching plan is still followed)."""
    wl = get_workload("video_dit_119k")
    q, k, v = (to_device_bf16(video119k[n]) for n in "qkv")
    r = sa.SolAttention(wl.B, wl.H, wl.N, wl.d)
    sa.pool(k, v, kpool=r.kpool, vmean=r.vmean)
    for plan_tau, tau in ((2.0, 8.0), (8.0, 2.0), (2.0, 2.0)):
        ref = r(q, k, v, tau, flags=sa.SOL_F_POOLED).clone()
        ref_stats = r.read_stats()
        r.plan(q, plan_tau)
        out = r(q, k, v, tau, flags=sa.SOL_F_POOLED | sa.SOL_F_PLANNED)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), (plan_tau, tau)
        assert r.read_stats() == ref_stats
        print(f"[plan] video_dit_119k plan at tau={plan_tau}, forward at tau={tau}: identical to unplanned",
              flush=True)


def test_garbage_workspace_is_reset():
    wl = _custom(1000, 128, H=3, seed=21)
    x = make_inputs(wl)
    q, k, v = (to_device_bf16(x[n]) for n in "qkv")
    r = sa.SolAttention(wl.B, wl.H, wl.N, wl.d)
    ref = r(q, k, v, 2.0).clone()
    stats = r.read_stats()
    r.workspace.fill_(-1)  # every byte 0xff
    out = r(q, k, v, 2.0)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    assert r.read_stats() == stats


@pytest.mark.parametrize("wlname,tau", [("video_dit_32k_imbalance", 8.0), ("video_dit_32k", 8.0), ("image_dit_4k", 2.0)])
def test_every_row_written(wlname, tau):
    """Outputs start as NaN: every row of every item must be written, whatever
    order the planning step picks (outliers first, the rest in sequence)."""
    wl = get_workload(wlname)
    x = make_inputs(wl)
    q, k, v = (to_device_bf16(x[n]) for n in "qkv")
    r = sa.SolAttention(wl.B, wl.H, wl.N, wl.d)
    out = torch.full((wl.B, wl.H, wl.N, wl.d), float("nan"), dtype=torch.float32, device=q.device)
    r(q, k, v, tau, out=out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    st = r.read_stats()
    assert st["total_blocks"] == wl.B * wl.H * wl.Nq * wl.Nk


# ---------------------------------------------------------------------------
# Gaussian-calibrated threshold and forced-keep sink blocks
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("beta", [-0.5, 0.5, 1.5, 3.0])
def test_gauss_rule_tiny(beta):
    _full_parity(get_workload("tiny_fp32"), 0.0, beta=beta)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 65, 1000])
@pytest.mark.parametrize("beta", [0.0, 2.0])
def test_gauss_rule_ragged(N, d, beta):
    _full_parity(_custom(N, d, H=2, seed=N + d + 7), 0.0, beta=beta)


def test_gauss_rule_image_and_video(video32k):
    _full_parity(get_workload("image_dit_4k"), 0.0, beta=2.0)
    _full_parity(get_workload("video_dit_32k"), 0.0, video32k, beta=3.0)


@pytest.mark.parametrize("sinks_at", ["start", "end"])
@pytest.mark.parametrize("N,d", [(1000, 64), (1000, 128), (130, 128)])
def test_sinks_rowmax(N, d, sinks_at):
    nk = -(-N // 64)
    sinks = (0, 2) if sinks_at == "start" else (nk - 2, 2)
    _full_parity(_custom(N, d, H=2, seed=N + 3), 0.0, sinks=sinks)
    _full_parity(_custom(N, d, H=2, seed=N + 3), 2.0, sinks=sinks)


def test_sinks_with_gauss_rule_and_exact_only():
    wl = get_workload("tiny_fp32")
    _full_parity(wl, 0.0, beta=1.0, sinks=(3, 2))
    x = make_inputs(wl)
    out, keep, _ = run_gpu(x["q"], x["k"], x["v"], 1.0, flags=sa.SOL_F_EXACT_ONLY, sinks=(0, 1))
    assert keep[..., 0].all()
    for h in range(wl.H):
        q, k, v = (bf16_bits_to_f64(x[n][0, h]) for n in "qkv")
        r = attend_head(q, k, v, 64, 64, 1.0, keep_override=keep[0, h], correction=False)
        assert np.abs(out[0, h] - r["out"]).max() <= 2e-2


def test_route_arguments_rejected():
    wl = _custom(1000, 128, H=1)
    x = make_inputs(wl)
    q, k, v = (to_device_bf16(x[n]) for n in "qkv")
    r = sa.SolAttention(1, 1, 1000, 128)
    for kw in (dict(beta=math.inf), dict(beta=math.nan), dict(sinks=(15, 2)), dict(sinks=(-1, 1)),
               dict(sinks=(0, -1))):
        with pytest.raises(sa.SolAttnError):
            r(q, k, v, 2.0, **kw)


# ---------------------------------------------------------------------------
# Token-to-block (per-row) correction
# ---------------------------------------------------------------------------

RC = sa.SOL_F_ROW_CORRECTION


@pytest.mark.parametrize("tau", [0.0, 2.0, 4.0, INF])
def test_row_correction_tiny(tau):
    _full_parity(get_workload("tiny_fp32"), tau, flags=RC)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 65, 130, 1000])
@pytest.mark.parametrize("tau", [0.0, 1.5])
def test_row_correction_ragged(N, d, tau):
    _full_parity(_custom(N, d, H=2, seed=N + d + 11), tau, flags=RC)


def test_row_correction_image_video_smooth(video32k):
    _full_parity(get_workload("image_dit_4k"), 2.0, flags=RC)
    _full_parity(get_workload("video_dit_32k"), 2.0, video32k, flags=RC)
    _full_parity(get_workload("video_dit_32k_smoothv"), 2.0, flags=RC)


def test_row_correction_with_gauss_and_sinks():
    _full_parity(get_workload("tiny_fp32"), 0.0, beta=1.0, sinks=(2, 2), flags=RC)
    _full_parity(_custom(1000, 128, H=2, seed=3), 1.0, sinks=(15, 1), flags=RC)


@pytest.mark.parametrize("d", [64, 128])
def test_row_correction_with_fully_kept_pooled_tiles(d):
    """Sinks over key blocks 0-63 make the first pooled tile one that every
    query block keeps whole (skipped by the kernel); the second tile and the
    ragged one-block third tile still carry corrections."""
    wl = _custom(8200, d, H=2, seed=21 + d)  # 129 key blocks: pooled tiles of 64, 64 and 1
    _full_parity(wl, 1.0, sinks=(0, 64), flags=RC, query_blocks_per_head=6, seed=21)


def test_row_correction_planned_matches_one_shot():
    wl = get_workload("image_dit_4k")
    x = make_inputs(wl)
    q, k, v = (to_device_bf16(x[n]) for n in "qkv")
    one = sa.SolAttention(wl.B, wl.H, wl.N, wl.d)
    ref = one(q, k, v, 2.0, flags=RC).clone()
    r = sa.SolAttention(wl.B, wl.H, wl.N, wl.d)
    sa.pool(k, v, kpool=r.kpool, vmean=r.vmean)
    r.plan(q, 2.0)
    out = r(q, k, v, 2.0, flags=RC | sa.SOL_F_POOLED | sa.SOL_F_PLANNED)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))


# ---------------------------------------------------------------------------
# Gaussian threshold with the diagonal estimator (threshold from pooled-key
# statistics, known before the proxy row)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("beta", [-0.5, 0.5, 2.0])
def test_gauss_diag_rule_tiny(beta):
    _full_parity(get_workload("tiny_fp32"), 0.0, beta=beta, diag=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 130, 1000])
def test_gauss_diag_rule_ragged(N, d):
    _full_parity(_custom(N, d, H=2, seed=N + d + 13), 0.0, beta=1.0, diag=True)


def test_gauss_diag_rule_video(video32k):
    _full_parity(get_workload("image_dit_4k"), 0.0, beta=1.5, diag=True)
    _full_parity(get_workload("video_dit_32k"), 0.0, video32k, beta=3.0, diag=True,
                 sinks=(0, 1), flags=sa.SOL_F_ROW_CORRECTION)


def test_order_never_changes_the_result():
    """The default call, a planned workspace with the identity order (a plan
    at tau = +inf) and ones planned at tau = 2 and 8 give the same bits."""
    wl = get_workload("image_dit_4k")
    x = make_inputs(wl)
    q, k, v = (to_device_bf16(x[n]) for n in "qkv")
    r = sa.SolAttention(wl.B, wl.H, wl.N, wl.d)
    ref = r(q, k, v, 8.0).clone()
    st = r.read_stats()
    for plan_tau in (INF, 2.0, 8.0):
        r.plan(q, plan_tau)
        out = r(q, k, v, 8.0, flags=sa.SOL_F_POOLED | sa.SOL_F_PLANNED)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), plan_tau
        assert r.read_stats() == st


@pytest.mark.parametrize("case", [
    ("tiny_fp32", None, 2.0, {}),
    ("custom", (130, 64), 0.0, {}),
    ("custom", (1000, 128), 4.0, dict(flags=sa.SOL_F_ROW_CORRECTION)),
    ("custom", (1000, 128), 0.0, dict(beta=0.5, sinks=(0, 2))),
    ("image_dit_4k", None, 8.0, {}),
    ("image_dit_4k", None, INF, {}),
])
def test_bf16_output_is_the_fp32_output_rounded(case):
    """SOL_F_OUT_BF16 stores the same fp32 result rounded to nearest even."""
    name, arg, tau, kw = case
    wl = get_workload(name) if arg is None else _custom(*arg)
    x = make_inputs(wl)
    q, k, v = (to_device_bf16(x[n]) for n in "qkv")
    r = sa.SolAttention(wl.B, wl.H, wl.N, wl.d)
    ref = r(q, k, v, tau, **kw).clone()
    st = r.read_stats()
    out16 = torch.full(ref.shape, float("nan"), dtype=torch.bfloat16, device=ref.device)
    got = r(q, k, v, tau, out=out16, **kw)
    torch.cuda.synchronize()
    assert got.dtype == torch.bfloat16
    assert torch.equal(got.view(torch.int16), ref.to(torch.bfloat16).view(torch.int16))
    assert r.read_stats() == st
    with pytest.raises(ValueError):
        r(q, k, v, tau, out=ref, flags=sa.SOL_F_OUT_BF16 | kw.get("flags", 0),
          **{a: b for a, b in kw.items() if a != "flags"})
