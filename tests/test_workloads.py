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


def test_pairs_counts_admitted_keys():
    """pairs() equals a direct count of (query, key) pairs admitted by the top-left rule."""
    from workloads import Workload

    for (n, nk) in ((5, 5), (5, 9), (9, 5), (1, 7), (7, 1)):
        for causal in (False, True):
            w = Workload("t", 1, 1, n, 16, "f32", causal, seed=0, Nk=nk if nk != n else 0)
            count = sum(1 for i in range(n) for j in range(nk) if not causal or j <= i)
            assert w.pairs() == count, (n, nk, causal)


def test_cross_workload_shapes():
    w = WORKLOADS["cross_bf16_b4h16q1024k4096d128"]
    q, k, v = w.make()
    assert q.shape == (4, 16, 1024, 128) and k.shape == v.shape == (4, 16, 4096, 128)
    assert w.io_bytes() == 2 * (4 * 16 * (1024 + 4096)) * 128 * 2 + 4 * 4 * 16 * 1024
