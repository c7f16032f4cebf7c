"""Benchmark of the Sol-Attn sparse attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--tau T]

A step is one full pass of the hot path over the video-DiT layer
(B=1, H=12, 21x30x52 grid -> N=32760, d=128, bf16 inputs resident in HBM):
the pooling pre-pass plus the fused routing / exact / correction kernel, one
C-ABI call; where the default call plans its work order (row-max rule,
tau >= 8 on this layer) it includes the planning kernels, which are also timed
on their own. The headline tau is 8; taus 2, 4 and +inf (the same kernel run
dense) are reported alongside. Prints ONE JSON line.

value = dense-equivalent TFLOP/s = 4*B*H*N^2*d / (seconds per call).
roofline = the fused kernel's own HIP-event time against the bf16 MFMA peak
(kept work) or the HBM peak (its algorithmic bytes), whichever floor is higher.
cpu_baseline = the fp64 oracle on this host's cores over whole heads, until
a time budget is spent (the full call when it fits), scaled to a full call.
parity = the GPU output and kept-block bitmap of the headline call compared
with that same oracle run, head by head (the routing exact away from a 1e-3
band around the threshold, the output within 2e-2 with the oracle following
the GPU's decisions inside the band).
per_workload = the other synthetic layers (tiny fp32 layer, 4K image layer,
imbalance layer, 119K video layer) at their taus: ms per call, kept blocks,
and the fused kernel against its binding roofline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import re
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
HEADLINE_TAU = 8.0
METRIC = "sparse-attn ms/call + dense-equiv TFLOP/s at N=32760,d=128; kept-block %"
KERNEL_SOURCES = ["block_sparse_attention_14_amd/csrc/fwd.hip", "block_sparse_attention_14_amd/csrc/common.h",
                  "block_sparse_attention_14_amd/csrc/kernels.h"]  # the fused kernel's sources
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_traffic_video_dit_32k_tau8.json")
BITMAP_TIE = 1e-3   # routing decisions closer than this to the threshold may go either way
OUT_ATOL = 2e-2     # output bar (bf16 inputs, fp32 accumulation, unit-scale outputs)
# the other layers measured beside the headline, with their taus
OTHER_WORKLOADS = (("tiny_fp32", (0.0, 2.0, 4.0, math.inf)),
                   ("image_dit_4k", (2.0, 4.0, 8.0)),
                   ("video_dit_32k_imbalance", (8.0,)),
                   ("video_dit_119k", (2.0, 4.0, 8.0)))


def kernel_hash() -> str:
    """Hash of the fused kernel's code with comments and whitespace removed, so
    that measured counters stay attached to it through comment-only edits."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="video_dit_32k")
    ap.add_argument("--tau", type=float, default=HEADLINE_TAU)
    ap.add_argument("--taus", default="2,4,8,inf", help="taus reported alongside the headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="time budget of the oracle baseline")
    ap.add_argument("--profile-only", action="store_true",
                    help="headline tau only, the fused kernel only in default calls and split stages (for profilers)")
    ap.add_argument("--no-ablation", action="store_true", help="skip the correction ablation report")
    ap.add_argument("--no-routing-cost", action="store_true", help="skip the router comparison")
    ap.add_argument("--no-rules", action="store_true", help="skip the Gaussian-rule and sink timings")
    ap.add_argument("--no-workloads", action="store_true", help="skip the per-workload lines")
    ap.add_argument("--workload-steps", type=int, default=10, help="timed calls per (workload, tau) line")
    ap.add_argument("--copy-ref-mib", type=int, default=512,
                    help="size of the plain device copy (reference rate, counter calibration, flush buffer)")
    return ap.parse_args(argv)


def tau_key(tau: float) -> str:
    return "inf" if math.isinf(tau) else f"{tau:g}"


def pct(xs):
    return {"median": round(float(np.median(xs)), 4), "p10": round(float(np.percentile(xs, 10)), 4),
            "p90": round(float(np.percentile(xs, 90)), 4)}


def fwd_roofline(B, H, N, d, Nk, stats, kv_tokens, ms_fwd, out_bytes=4):
    """The fused kernel's algorithmic work and which floor binds it.

    flops: 4 d sum_kept n_i n_j (QK^T and PV over the kept pairs, from the stats).
    bytes: q read once, K and V of every key block kept by some query block read
    once, the output written once, the pooled keys and values read once."""
    flops = 4.0 * d * stats["kept_pairs"]
    nbytes = (B * H * N * d * 2 + 2 * kv_tokens * d * 2 + B * H * N * d * out_bytes + 2 * B * H * Nk * d * 4)
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    mfma_frac = flops / (ms_fwd * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS
    hbm_frac = nbytes / (ms_fwd * 1e-3) / 1e9 / HBM_PEAK_GBS
    return {"flops": flops, "bytes": nbytes, "bound": "mfma" if t_mfma >= t_hbm else "hbm",
            "mfma_frac": mfma_frac, "hbm_frac": hbm_frac}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py runs on one GPU only: the sparse forward shards per (batch, head) with no "
              f"exchange, so a multi-GPU figure is one GPU's work repeated; --gpus {args.gpus} is not run.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import block_sparse_attention_14_amd as sa
    from workloads import get_workload, make_inputs

    wl = get_workload(args.workload)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    t0 = time.perf_counter()
    x = make_inputs(wl)
    gen_s = time.perf_counter() - t0
    q, k, v = (torch.from_numpy(x[n].view(np.int16)).to(dev).view(torch.bfloat16) for n in "qkv")
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    runner = sa.SolAttention(B, H, N, d, dev)
    out = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    dense = wl.dense_flops()
    stream = torch.cuda.current_stream(dev)

    # a plain device copy of known size: the reference rate for the pool pass,
    # and (when profiling) the calibration of the traffic counters
    copy_mib = args.copy_ref_mib or 512
    src = torch.ones(copy_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() * 4 * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del dst
    scratch = src  # rewritten between calls of the flushed run (evicts L2 and the MALL)

    def events(n):
        return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]

    def elapsed(ev):
        return [a.elapsed_time(b) for a, b in ev]

    def timed_calls(fn, n):
        ev = events(n)
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return elapsed(ev)

    def split_calls(rn, qq, kk, vv, oo, tau, n):
        """The call's stages timed one by one: the pool pass of k and v, the
        forward's pre-pass (pooled queries, routing planes), the planning
        kernels (item costs, queue order), then the fused kernel alone in the
        planned order (HIP events on the stream it runs on)."""
        ev1, ev2, ev3, ev4 = events(n), events(n), events(n), events(n)
        for (a, b), (c, e), (f, g), (h, i) in zip(ev1, ev2, ev3, ev4):
            a.record(stream)
            sa.pool(kk, vv, kpool=rn.kpool, vmean=rn.vmean)
            b.record(stream)
            c.record(stream)
            rn.prepare(qq)
            e.record(stream)
            f.record(stream)
            rn.plan(qq, tau)
            g.record(stream)
            h.record(stream)
            rn(qq, kk, vv, tau, out=oo, flags=sa.SOL_F_POOLED | sa.SOL_F_PREPARED | sa.SOL_F_PLANNED)
            i.record(stream)
        torch.cuda.synchronize()
        return elapsed(ev1), elapsed(ev2), elapsed(ev3), elapsed(ev4)

    def kv_unique_tokens(rn, qq, kk, vv, oo, tau, w):
        """Tokens of the key blocks kept by at least one query block of their
        head (from the exported bitmap), and the bitmap itself."""
        bm = torch.zeros(sa.bitmap_shape(w.B, w.H, w.N), dtype=torch.int32, device=dev)
        rn(qq, kk, vv, tau, out=oo, bitmap=bm)
        torch.cuda.synchronize()
        keep = sa.unpack_bitmap(bm, w.Nk)  # [B, H, Nq, Nk]
        used = keep.any(axis=2)            # [B, H, Nk]
        n = np.minimum(64, w.N - 64 * np.arange(w.Nk))
        return int((used * n[None, None, :]).sum()), keep

    def measure(tau: float, steps: int, warmup: int):
        for _ in range(warmup):
            runner(q, k, v, tau, out=out)
        torch.cuda.synchronize()
        # the timed steps: one C-ABI call (pool + fused) each, inputs resident in HBM
        t_wall = time.perf_counter()
        r = {"call": timed_calls(lambda: runner(q, k, v, tau, out=out), steps)}
        wall = time.perf_counter() - t_wall
        # (with --profile-only the fused kernel runs only as the default call and
        # the split stages time it: a kernel trace's average is then the figure
        # the roofline uses)
        extras = not args.profile_only
        if extras:
            # the same calls with L2 and the MALL flushed first
            ev = events(steps)
            for i, (a, b) in enumerate(ev):
                scratch.fill_(float(i))
                a.record(stream)
                runner(q, k, v, tau, out=out)
                b.record(stream)
            torch.cuda.synchronize()
            r["call_flushed"] = elapsed(ev)
        r["pool"], r["prepare"], r["plan"], r["fwd"] = split_calls(runner, q, k, v, out, tau, steps)
        stats = runner.read_stats()
        if not extras:
            return r, wall, stats
        n = max(3, steps // 2)
        # the fused kernel with its items in sequence (the identity order)
        runner.plan(q, math.inf)
        r["fwd_sequence_order"] = timed_calls(
            lambda: runner(q, k, v, tau, out=out, flags=sa.SOL_F_POOLED | sa.SOL_F_PREPARED | sa.SOL_F_PLANNED), n)
        # the whole call with the token-to-block (per-row) correction
        r["call_row_correction"] = timed_calls(lambda: runner(q, k, v, tau, out=out, flags=sa.SOL_F_ROW_CORRECTION), n)
        # the whole call with the output stored as bf16 (SOL_F_OUT_BF16)
        out16 = torch.empty(out.shape, dtype=torch.bfloat16, device=out.device)
        r["call_bf16_out"] = timed_calls(lambda: runner(q, k, v, tau, out=out16), n)
        return r, wall, stats

    taus = [args.tau] if args.profile_only else sorted(
        {args.tau} | {math.inf if t.strip() == "inf" else float(t) for t in args.taus.split(",")})
    per_tau = {}
    head = None
    for tau in taus:
        steps = args.steps if tau == args.tau else max(3, args.steps // 2)
        r, wall, stats = measure(tau, steps, args.warmup if tau == args.tau else 2)
        ms_call = float(np.mean(r["call"]))
        ms_pool, ms_prep, ms_plan, ms_fwd = (float(np.median(r[x_])) for x_ in ("pool", "prepare", "plan", "fwd"))
        kv_tokens, _ = kv_unique_tokens(runner, q, k, v, out, tau, wl)
        rl = fwd_roofline(B, H, N, d, wl.Nk, stats, kv_tokens, ms_fwd)
        kept_pct = 100.0 * stats["kept_blocks"] / stats["total_blocks"]

        def med(key):
            return round(float(np.median(r[key])), 4) if key in r else None

        rec = {
            "ms_per_call": round(ms_call, 4),
            "call_ms": pct(r["call"]),
            "call_ms_l2_mall_flushed": pct(r["call_flushed"]) if "call_flushed" in r else None,
            "ms_pool": round(ms_pool, 4),
            "ms_prepare": round(ms_prep, 4),
            "ms_fwd": round(ms_fwd, 4),
            "fwd_ms": pct(r["fwd"]),
            "ms_plan": round(ms_plan, 4),
            "fwd_ms_items_in_sequence": med("fwd_sequence_order"),
            "row_correction_ms_per_call": med("call_row_correction"),
            "bf16_out_ms_per_call": med("call_bf16_out"),
            "dense_equiv_tflops": round(dense / (ms_call * 1e-3) / 1e12, 1),
            "kept_block_pct": round(kept_pct, 3),
            "kept_token_pct": round(100.0 * stats["kept_pairs"] / (B * H * N * N), 3),
            "kept_per_query_block_min_max": [stats["min_kept"], stats["max_kept"]],
            "fwd_mfma_frac_of_peak": round(rl["mfma_frac"], 4),
            "fwd_hbm_frac_of_peak": round(rl["hbm_frac"], 4),
            "fwd_floor_bound": rl["bound"],
            "pool_gbs": round((2 * B * H * N * d * 2 + 2 * B * H * wl.Nk * d * 4) / (ms_pool * 1e-3) / 1e9, 1),
        }
        per_tau[tau_key(tau)] = rec
        print(f"[bench] tau={tau:g} {json.dumps(rec)}", file=sys.stderr, flush=True)
        if tau == args.tau:
            head = (ms_call, ms_pool, ms_fwd, stats, rl, kept_pct, steps)

    ms_call, ms_pool, ms_fwd, stats, rl, kept_pct, steps = head
    if rl["bound"] == "mfma":
        achieved, peak, unit = rl["flops"] / (ms_fwd * 1e-3) / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = rl["bytes"] / (ms_fwd * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_hash") == kernel_hash() and args.workload == "video_dit_32k" and args.tau == 8.0:
            traffic = tr.get("bytes_per_launch")

    # the headline call's own output and routing, kept for the parity witness
    head_bm = torch.zeros(sa.bitmap_shape(B, H, N), dtype=torch.int32, device=dev)
    runner(q, k, v, args.tau, out=out, bitmap=head_bm)
    torch.cuda.synchronize()
    head_out = out.cpu().numpy()
    head_keep = sa.unpack_bitmap(head_bm, wl.Nk)
    del head_bm

    def ablation(wname, taus_ab):
        """Block-level corrected, per-row corrected and exact-only outputs for
        the same routing, against this kernel's dense (tau = +inf) output:
        global relative L2 error and the mean cosine similarity of rows."""
        wl2 = get_workload(wname)
        x2 = make_inputs(wl2)
        q2, k2, v2 = (torch.from_numpy(x2[n].view(np.int16)).to(dev).view(torch.bfloat16) for n in "qkv")
        r2 = sa.SolAttention(wl2.B, wl2.H, wl2.N, wl2.d, dev)
        dense_out = r2(q2, k2, v2, math.inf).double()
        dn = dense_out.norm()

        def metrics(o):
            o = o.double()
            cos = torch.nn.functional.cosine_similarity(o.reshape(-1, wl2.d), dense_out.reshape(-1, wl2.d), dim=1)
            return {"rel_l2": round(float((o - dense_out).norm() / dn), 5), "cos": round(float(cos.mean()), 5)}

        rep_ = {}
        for tau in taus_ab:
            c = metrics(r2(q2, k2, v2, tau))
            kept = r2.read_stats()
            e = metrics(r2(q2, k2, v2, tau, flags=sa.SOL_F_EXACT_ONLY))
            rc = metrics(r2(q2, k2, v2, tau, flags=sa.SOL_F_ROW_CORRECTION))
            rep_[f"{tau:g}"] = {"kept_block_pct": round(100.0 * kept["kept_blocks"] / kept["total_blocks"], 3),
                                "corrected": c, "row_corrected": rc, "exact_only": e}
        del q2, k2, v2, r2, dense_out
        torch.cuda.empty_cache()
        return rep_

    def routing_cost(tau, kept_blocks):
        """The kept-block bitmap from three routers on the same layer: on-chip
        threshold routing (no proxy map) against top-k and top-p, which pool q,
        write the full proxy map to device memory and sort each row. top-k is
        given the threshold rule's mean budget."""
        mb = sa.MaskBuilder(B, H, N, d, dev)
        kp, _ = sa.pool(k, v)
        kk = max(1, round(kept_blocks / (B * H * wl.Nq)))

        def timed(fn, n=10):
            fn()
            torch.cuda.synchronize()
            return float(np.median(timed_calls(fn, n)))

        res = {}
        for name, fn in (("threshold_on_chip", lambda: mb.threshold(q, kp, tau=tau)),
                         ("topk_proxy_map", lambda: mb.topk(q, kp, kk)),
                         ("topp_proxy_map", lambda: mb.topp(q, kp, 0.9))):
            ms = timed(fn)
            kept = int(sa.unpack_bitmap(mb.bitmap, wl.Nk).sum())
            res[name] = {"ms": round(ms, 4), "kept_block_pct": round(100.0 * kept / (B * H * wl.Nq * wl.Nk), 3)}
        res["topk_proxy_map"]["k"] = kk
        res["topp_proxy_map"]["p"] = 0.9
        res["proxy_map_bytes"] = B * H * wl.Nq * wl.Nk * 4
        t0_ = res["threshold_on_chip"]["ms"]
        res["speedup_vs_topk"] = round(res["topk_proxy_map"]["ms"] / t0_, 2)
        res["speedup_vs_topp"] = round(res["topp_proxy_map"]["ms"] / t0_, 2)
        res["tau"] = tau
        del mb
        torch.cuda.empty_cache()
        return res

    def rules_report(tau):
        """Whole calls with the Gaussian-calibrated thresholds (moments of the
        on-chip proxy row, and the diagonal estimator from pooled-key
        statistics) at three cutoffs, and with the row-max rule plus four
        forced sink blocks, on the same layer."""
        def timed(fn, n=10):
            fn()
            torch.cuda.synchronize()
            return float(np.median(timed_calls(fn, n)))

        res = {}
        for diag in (False, True):
            for beta in (1.0, 2.0, 3.0):
                ms = timed(lambda: runner(q, k, v, 0.0, out=out, beta=beta, diag=diag))
                st = runner.read_stats()
                res[f"{'gauss_diag' if diag else 'gauss'}_beta{beta:g}"] = {
                    "ms_per_call": round(ms, 4),
                    "kept_block_pct": round(100.0 * st["kept_blocks"] / st["total_blocks"], 3)}
        ms = timed(lambda: runner(q, k, v, tau, out=out, sinks=(0, 4)))
        st = runner.read_stats()
        res[f"rowmax_tau{tau:g}_sinks_0_4"] = {"ms_per_call": round(ms, 4),
                                              "kept_block_pct": round(100.0 * st["kept_blocks"] / st["total_blocks"], 3)}
        return res

    def workload_lines():
        """Each other layer at its taus: the whole call (events around it), the
        fused kernel alone (planned workspace), kept blocks, and the fused
        kernel's fraction of its binding roofline."""
        res = {}
        for wname, wtaus in OTHER_WORKLOADS:
            w = get_workload(wname)
            t_gen = time.perf_counter()
            xw = make_inputs(w)
            t_gen = time.perf_counter() - t_gen
            qw, kw, vw = (torch.from_numpy(xw[n].view(np.int16)).to(dev).view(torch.bfloat16) for n in "qkv")
            del xw
            rw = sa.SolAttention(w.B, w.H, w.N, w.d, dev)
            ow = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device=dev)
            lines = {}
            for tau in wtaus:
                for _ in range(2):
                    rw(qw, kw, vw, tau, out=ow)
                torch.cuda.synchronize()
                call = timed_calls(lambda: rw(qw, kw, vw, tau, out=ow), args.workload_steps)
                _, _, _, fwd = split_calls(rw, qw, kw, vw, ow, tau, args.workload_steps)
                st = rw.read_stats()
                kv_tok, _ = kv_unique_tokens(rw, qw, kw, vw, ow, tau, w)
                ms_c, ms_f = float(np.mean(call)), float(np.median(fwd))
                rlw = fwd_roofline(w.B, w.H, w.N, w.d, w.Nk, st, kv_tok, ms_f)
                lines[tau_key(tau)] = {
                    "ms_per_call": round(ms_c, 4),
                    "call_ms": pct(call),
                    "ms_fwd": round(ms_f, 4),
                    "dense_equiv_tflops": round(w.dense_flops() / (ms_c * 1e-3) / 1e12, 1),
                    "kept_block_pct": round(100.0 * st["kept_blocks"] / st["total_blocks"], 3),
                    "kept_per_query_block_min_max": [st["min_kept"], st["max_kept"]],
                    "fwd_bound": rlw["bound"],
                    "fwd_frac_of_bound": round(rlw["mfma_frac"] if rlw["bound"] == "mfma" else rlw["hbm_frac"], 4),
                    "fwd_mfma_frac_of_peak": round(rlw["mfma_frac"], 4),
                    "fwd_hbm_frac_of_peak": round(rlw["hbm_frac"], 4),
                }
                print(f"[bench] {wname} tau={tau:g} {json.dumps(lines[tau_key(tau)])}", file=sys.stderr, flush=True)
            res[wname] = {"B": w.B, "H": w.H, "N": w.N, "d": w.d, "grid_thw": list(w.grid),
                          "input_generation_s": round(t_gen, 2), "taus": lines}
            del qw, kw, vw, rw, ow
            torch.cuda.empty_cache()
        return res

    rules = None
    if not args.no_rules and not args.profile_only:
        rules = rules_report(args.tau)
        print(f"[bench] rules {json.dumps(rules)}", file=sys.stderr, flush=True)

    rcost = None
    if not args.no_routing_cost and not args.profile_only:
        rcost = routing_cost(args.tau, stats["kept_blocks"])
        print(f"[bench] routing_cost {json.dumps(rcost)}", file=sys.stderr, flush=True)

    abl = None
    if not args.no_ablation and not args.profile_only:
        abl = {"reference": "this kernel at tau = +inf (dense attention)",
               "video_dit_32k": ablation("video_dit_32k", (2.0, 4.0, 8.0)),
               "video_dit_32k_smoothv": ablation("video_dit_32k_smoothv", (2.0, 4.0, 8.0)),
               "video_dit_32k_mild": ablation("video_dit_32k_mild", (1.0, 2.0, 4.0))}
        print(f"[bench] ablation {json.dumps(abl)}", file=sys.stderr, flush=True)

    per_wl = None
    if not args.no_workloads and not args.profile_only:
        per_wl = workload_lines()

    cpu = parity = None
    if not args.no_cpu_baseline and not args.profile_only:
        cpu, parity = cpu_baseline(wl, x, args.tau, args.cpu_seconds, gpu_out=head_out, gpu_keep=head_keep)
        print(f"[bench] parity {json.dumps(parity)}", file=sys.stderr, flush=True)

    line = {
        "metric": METRIC,
        "value": round(dense / (ms_call * 1e-3) / 1e12, 1),
        "unit": "TFLOP/s (dense-equivalent, 4*B*H*N^2*d per call)",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_call, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "H": H, "grid_thw": list(wl.grid), "N": N, "d": d,
                   "Bq": wl.Bq, "Bk": wl.Bk, "tau": args.tau, "out_dtype": "fp32"},
        "ms_per_call": round(ms_call, 4),
        "kept_block_pct": round(kept_pct, 3),
        "ms_pool": round(ms_pool, 4),
        "ms_prepare": round(per_tau[tau_key(args.tau)]["ms_prepare"], 4),
        "ms_plan": round(per_tau[tau_key(args.tau)]["ms_plan"], 4),
        "ms_fwd": round(ms_fwd, 4),
        "pool_gbs": per_tau[tau_key(args.tau)]["pool_gbs"],
        "device_copy_gbs": round(copy_gbs, 1),
        "roofline": {
            "kernel": "fwd_kernel<128, G> (fused routing + kept MFMA + correction; G query blocks per work item, "
                      "chosen by the library); HIP events around the fused launch alone (prepared and planned "
                      "workspace)",
            "bound": rl["bound"],
            "achieved": round(achieved, 1),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "algorithmic_flops": rl["flops"],
            "algorithmic_bytes": rl["bytes"],
        },
        "cpu_baseline": cpu,
        "parity": parity,
        "correction_ablation": abl,
        "routing_cost": rcost,
        "routing_rules": rules,
        "per_tau": per_tau,
        "per_workload": per_wl,
        "context": {
            "pages_end_to_end_speedup_video_generation": "2.1x vs dense attention (hardware not stated)",
            "pages_end_to_end_speedup_video_editing": "2.3x vs dense attention (hardware not stated)",
        },
        "input_generation_s": round(gen_s, 2),
    }
    print(json.dumps(line), flush=True)


def cpu_model() -> str:
    """The host CPU's model name, as lscpu reports it (else /proc/cpuinfo);
    a name without a model number (some virtual machines report only the
    brand) gets lscpu's CPU family, model and stepping appended."""
    try:
        r = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20)
        fields = {}
        for ln in r.stdout.splitlines():
            if ":" in ln:
                key, val = ln.split(":", 1)
                fields.setdefault(key.strip().lower(), val.strip())
        name = fields.get("model name")
        if name:
            if not any(ch.isdigit() for ch in name):
                ids = [f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if fields.get(k)]
                if ids:
                    name += " (" + ", ".join(ids) + ")"
            return name
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def usable_cores() -> int:
    """Cores this process may run on (its CPU affinity set)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def compare_head(out_gpu, keep_gpu, q, k, v, ref, Bq, Bk, tau):
    """One head of the GPU result against the oracle's run of it.

    Routing: every decision must agree except where the oracle's proxy lies
    within BITMAP_TIE of the threshold M - tau (either decision is right
    there). Output: max |gpu - oracle| over every row, with the oracle redone,
    following the GPU's routing, on the query blocks whose routing differs
    inside that band. Returns (max abs error, decisions differing outside the
    band, decisions differing inside it)."""
    from oracle import attend_head

    s, M = ref["s"], ref["M"]
    diff = keep_gpu != ref["keep"]
    if math.isinf(tau):
        near = np.zeros_like(diff)
    else:
        near = np.abs(s - (M - tau)[:, None]) <= BITMAP_TIE
    outside = int((diff & ~near).sum())
    ref_out = ref["out"]
    redo = np.flatnonzero(diff.any(axis=1))
    if len(redo):
        r2 = attend_head(q, k, v, Bq, Bk, tau, keep_override=keep_gpu, query_blocks=redo)
        ref_out = ref_out.copy()
        for i in redo:
            ref_out[i * Bq:min(q.shape[0], (i + 1) * Bq)] = r2["out"][i * Bq:min(q.shape[0], (i + 1) * Bq)]
    err = float(np.abs(out_gpu - ref_out).max()) if np.isfinite(out_gpu).all() else math.inf
    return err, outside, int((diff & near).sum())


def cpu_baseline(wl, x, tau, budget_s, gpu_out=None, gpu_keep=None):
    """The fp64 oracle timed on this host: whole heads, in a seeded order,
    until the time budget is spent (every head when it fits), scaled to a
    full call. The BLAS pool is set to every usable core. With the GPU's
    output and bitmap given, every head the oracle ran is also compared with
    them (the comparison is outside the timed region).

    Returns (cpu_baseline record, parity record or None)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import attend_head
    from workloads import bf16_bits_to_f64

    cores = usable_cores()
    rng = np.random.default_rng(123)
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    rng.shuffle(heads)
    done = 0
    t_total = 0.0
    worst, outside, inside = 0.0, 0, 0
    with threadpool_limits(limits=cores, user_api="blas"):
        threads = sum(p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas") or 1
        for b, h in heads:
            qh, kh, vh = (bf16_bits_to_f64(x[n][b, h]) for n in "qkv")
            t0 = time.perf_counter()
            ref = attend_head(qh, kh, vh, wl.Bq, wl.Bk, tau)
            t_total += time.perf_counter() - t0
            done += 1
            if gpu_out is not None:
                e, o, i = compare_head(gpu_out[b, h], gpu_keep[b, h], qh, kh, vh, ref, wl.Bq, wl.Bk, tau)
                worst, outside, inside = max(worst, e), outside + o, inside + i
            if t_total > budget_s:
                break
    full_s = t_total / done * len(heads)
    what = "the full call" if done == len(heads) else f"{done} of {len(heads)} heads (seeded order), " \
                                                      f"extrapolated linearly to the full call"
    rec = {
        "value": round(wl.dense_flops() / full_s / 1e12, 4),
        "unit": "TFLOP/s (dense-equivalent, 4*B*H*N^2*d per call)",
        "ms_per_call": round(full_s * 1e3, 1),
        "cores": threads,
        "usable_cores": cores,
        "kind": "oracle",
        "sample": f"{what} at tau={tau:g}: {t_total:.1f} s of fp64 oracle time (numpy, {threads} BLAS threads)",
        "host_cpu": cpu_model(),
    }
    par = None
    if gpu_out is not None:
        par = {
            "reference": "the fp64 oracle run of cpu_baseline, on the same bf16 inputs",
            "heads_checked": done,
            "heads_total": len(heads),
            "rows_checked": done * wl.N,
            "max_abs_err": round(worst, 6) if math.isfinite(worst) else None,
            "out_atol": OUT_ATOL,
            "bitmap_mismatch_outside_band": outside,
            "bitmap_mismatch_inside_band": inside,
            "band": BITMAP_TIE,
            "pass": bool(math.isfinite(worst) and worst <= OUT_ATOL and outside == 0),
        }
    return rec, par


if __name__ == "__main__":
    main()
