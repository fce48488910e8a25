"""The seeded input generator: deterministic, right shapes, types and spreads (CPU)."""

import math

import torch

from workloads import HEADLINE, WORKLOADS, default_scale, make_qkv, sample_rows


def test_generation_is_deterministic_and_seed_dependent():
    a = make_qkv(1, 2, 33, 64, "bf16", seed=9)
    b = make_qkv(1, 2, 33, 64, "bf16", seed=9)
    c = make_qkv(1, 2, 33, 64, "bf16", seed=10)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert not torch.equal(a[0], c[0])


def test_shapes_types_and_spread():
    q, k, v = make_qkv(2, 3, 500, 128, "bf16", seed=5, sigma_qk=4.0)
    for t in (q, k, v):
        assert t.shape == (2, 3, 500, 128) and t.dtype == torch.bfloat16 and t.is_contiguous()
    assert abs(q.float().std().item() - 4.0) < 0.1
    assert abs(v.float().std().item() - 1.0) < 0.03
    q32, _, _ = make_qkv(1, 1, 64, 64, "f32", seed=1)
    assert q32.dtype == torch.float32


def test_bf16_inputs_are_rne_casts_of_the_fp32_draw():
    q16, _, _ = make_qkv(1, 1, 64, 64, "bf16", seed=3)
    q32, _, _ = make_qkv(1, 1, 64, 64, "f32", seed=3)
    assert torch.equal(q16, q32.to(torch.bfloat16))


def test_workload_table():
    assert set(WORKLOADS) >= {HEADLINE}
    w = WORKLOADS[HEADLINE]
    assert (w.B, w.H, w.N, w.d, w.dtype, w.causal) == (4, 16, 4096, 128, "bf16", True)
    assert w.flops() == 4 * 4 * 16 * 128 * (4096 * 4097 // 2)
    assert default_scale(128) == torch.tensor(1 / math.sqrt(128), dtype=torch.float32).item()
    r = sample_rows(1000, 16, seed=5)
    assert r[0] == 0 and r[-1] == 999 and len(r) == 16 and len(set(r)) == 16
