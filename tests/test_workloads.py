"""The seeded input generators: determinism, shapes, position code, rounding."""
import math

import numpy as np
import pytest
import torch

from workloads import (
    WORKLOADS,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    get_workload,
    make_head,
    make_inputs,
    pos_code,
)


def test_workload_shapes():
    expect = {
        "tiny_fp32": (1, 2, 1024, 64, 16),
        "image_dit_4k": (2, 24, 4096, 128, 64),
        "video_dit_32k": (1, 12, 32760, 128, 512),
        "video_dit_32k_imbalance": (1, 12, 32760, 128, 512),
        "video_dit_32k_smoothv": (1, 12, 32760, 128, 512),
        "video_dit_32k_mild": (1, 12, 32760, 128, 512),
        "video_dit_119k": (1, 24, 118800, 128, 1857),
    }
    for name, (B, H, N, d, Nq) in expect.items():
        w = get_workload(name)
        assert (w.B, w.H, w.N, w.d, w.Nq, w.Nk) == (B, H, N, d, Nq, Nq)
    assert get_workload("video_dit_32k").N - 511 * 64 == 56
    assert get_workload("video_dit_119k").N - 1856 * 64 == 16


@pytest.mark.parametrize("d", [64, 128])
def test_pos_code_norm_and_split(d):
    P = pos_code((3, 4, 5), d)
    assert P.shape == (60, d)
    np.testing.assert_allclose(np.linalg.norm(P, axis=1), math.sqrt(d), rtol=1e-12)
    # tokens differing only in w share the t and h groups exactly
    g = 2 * (d // 6)
    np.testing.assert_array_equal(P[0, : 2 * g] / np.linalg.norm(P[0]), P[1, : 2 * g] / np.linalg.norm(P[1]))


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    x[:4] = [0.0, -0.0, 1.00390625, 1.01171875]  # exact ties: round to even
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generation_deterministic_and_per_head():
    w = get_workload("tiny_fp32")
    a = make_inputs(w)
    b = make_inputs(w)
    for n in "qkv":
        np.testing.assert_array_equal(a[n], b[n])
    one = make_inputs(w, heads=[(0, 1)])
    np.testing.assert_array_equal(one["q"][0, 1], a["q"][0, 1])
    assert not one["q"][0, 0].any()
    q, k, v = make_head(w, 0, 1)
    np.testing.assert_array_equal(f32_to_bf16_bits(k), a["k"][0, 1])


def test_imbalance_construction():
    w = get_workload("video_dit_32k_imbalance")
    assert [w.head_locality(h) for h in range(12)] == [3.0] * 6 + [0.0] * 6
    # diffuse heads carry no position code: q is plain N(0,1)
    q, k, v = make_head(w, 0, 7)
    assert abs(q.mean()) < 1e-2 and abs(q.std() - 1) < 1e-2
    # sink heads: the first 4 KV blocks are shifted by 2*mean(q)
    q0, k0, _ = make_head(w, 0, 0)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 0, 0])))
    rng.standard_normal((w.N, w.d), dtype=np.float32)
    k_raw = rng.standard_normal((w.N, w.d), dtype=np.float32)
    from workloads.gen import _pos32
    k_raw += np.float32(3.0) * _pos32(w.grid, w.d)
    shift = k0[:256] - k_raw[:256]
    np.testing.assert_allclose(shift, np.broadcast_to(2 * q0.astype(np.float64).mean(0), shift.shape), atol=1e-5)
    np.testing.assert_array_equal(k0[256:], k_raw[256:])


def test_all_workloads_registered():
    assert set(WORKLOADS) == {"tiny_fp32", "image_dit_4k", "video_dit_32k",
                              "video_dit_32k_imbalance", "video_dit_32k_smoothv", "video_dit_32k_mild",
                              "video_dit_119k"}


def test_smooth_values_share_the_position_code():
    from workloads.gen import make_head, pos_code

    w = get_workload("video_dit_32k_smoothv")
    q, k, v = make_head(w, 0, 0)
    P = pos_code(w.grid, w.d)
    # v = noise + 3 P: its projection on P is about 3 |P|^2 per token
    c = float((v.astype(np.float64) * P).sum() / (P * P).sum())
    assert abs(c - 3.0) < 0.05


def test_mild_layer_scales_the_draws():
    """video_dit_32k_mild: q and k are 0.5 N(0, 1) + 1.5 P(pos), v is N(0, 1) + 3 P(pos);
    the other layers keep unit draws (their generated bits are unchanged)."""
    from workloads.gen import _pos32, make_head

    w = get_workload("video_dit_32k_mild")
    q, k, v = make_head(w, 0, 3)
    P = _pos32(w.grid, w.d)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 0, 3])))
    zq = rng.standard_normal((w.N, w.d), dtype=np.float32)
    zk = rng.standard_normal((w.N, w.d), dtype=np.float32)
    zv = rng.standard_normal((w.N, w.d), dtype=np.float32)
    np.testing.assert_array_equal(q, np.float32(0.5) * zq + np.float32(1.5) * P)
    np.testing.assert_array_equal(k, np.float32(0.5) * zk + np.float32(1.5) * P)
    np.testing.assert_array_equal(v, zv + np.float32(3.0) * P)
    assert get_workload("video_dit_32k").qk_noise == 1.0
