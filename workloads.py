"""Seeded synthetic inputs for the attention forward pass.

Shared by the tests, the benchmark and the smoke check: it fixes shapes, seeds
and value distributions, and nothing else. It holds none of the attention
arithmetic and imports neither the oracle nor the HIP binding.

Recipe (every workload): a CPU ``torch.Generator`` seeded with the workload's
seed draws Q, then K, then V as float32 standard normals of shape [B, H, N, d]
(K and V [B, H, Nk, d] for a cross-attention workload);
Q and K are multiplied by ``sigma_qk``, V by ``sigma_v``; the three tensors are
then cast to the workload's element type (bf16 with round-to-nearest-even).
Both the oracle and the GPU path consume exactly those cast values. The score
multiplier is 1/sqrt(d) rounded to float32, the value the caller hands to the
kernel; the oracle widens that same float32 value.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "f32" or "bf16"
    causal: bool
    seed: int
    sigma_qk: float = 1.0
    sigma_v: float = 1.0
    Nk: int = 0  # key rows when they differ from the N query rows (0: Nk = N)

    @property
    def keys(self) -> int:
        return self.Nk or self.N

    @property
    def torch_dtype(self):
        return torch_dtype(self.dtype)

    @property
    def scale(self) -> float:
        return default_scale(self.d)

    def make(self):
        if self.Nk:
            return make_qkv_cross(self.B, self.H, self.N, self.Nk, self.d, self.dtype, self.seed,
                                  self.sigma_qk, self.sigma_v)
        return make_qkv(self.B, self.H, self.N, self.d, self.dtype, self.seed,
                        self.sigma_qk, self.sigma_v)

    def pairs(self) -> int:
        """(query, key) pairs that enter the softmax per head: N Nk, or, when causal,
        sum over queries i of min(i + 1, Nk) (N(N+1)/2 when Nk = N)."""
        n, nk = self.N, self.keys
        if not self.causal:
            return n * nk
        if nk >= n:
            return n * (n + 1) // 2
        return nk * (nk + 1) // 2 + (n - nk) * nk

    def flops(self) -> int:
        """Algorithmic FLOPs of the two contractions: 2d for Q.k plus 2d for p.v per pair."""
        return 4 * self.B * self.H * self.d * self.pairs()

    def io_bytes(self) -> int:
        """Algorithmic HBM bytes: read Q, K, V once, write O once and the fp32 L once."""
        esize = 2 if self.dtype == "bf16" else 4
        n = self.B * self.H * self.N
        nk = self.B * self.H * self.keys
        return 2 * (n + nk) * self.d * esize + 4 * n


WORKLOADS = {
    w.name: w
    for w in [
        # one head, non-causal, fp32, N=128, d=64
        Workload("single_head_f32", 1, 1, 128, 64, "f32", False, seed=1),
        # eight sequences of one head, non-causal, fp32, N=1024, d=64
        Workload("batch8_f32", 8, 1, 1024, 64, "f32", False, seed=2),
        # causal bf16, four sequences of sixteen heads, N=4096, d=128
        Workload("causal_bf16_b4h16n4096d128", 4, 16, 4096, 128, "bf16", True, seed=3),
        # long causal bf16, thirty-two heads, N=16384, d=64
        Workload("long_causal_bf16_h32n16384d64", 1, 32, 16384, 64, "bf16", True, seed=4),
        # ragged N=1000, non-causal bf16, wide logits: Q, K ~ N(0, 4^2), V ~ N(0, 1)
        Workload("ragged_wide_logits_bf16_n1000", 2, 8, 1000, 128, "bf16", False, seed=5,
                 sigma_qk=4.0),
        # cross-attention (through the strided entry point): 1024 queries over 4096 keys,
        # non-causal bf16, B=4, H=16, d=128
        Workload("cross_bf16_b4h16q1024k4096d128", 4, 16, 1024, 128, "bf16", False, seed=6, Nk=4096),
    ]
}

# The throughput workload: causal bf16, B=4, H=16, N=4096, d=128.
HEADLINE = "causal_bf16_b4h16n4096d128"

# The small-shape sweep of "Writing a FlashAttention kernel in Metal" (the benchmark
# section): fp32, one sequence and one head, N in {64, 256, 1024, 2048}, d in {32, 64},
# causal and not -- sixteen latency-bound configurations.
SMALL_SWEEP = [
    Workload(f"sweep_f32_n{n}_d{d}_{'causal' if causal else 'full'}", 1, 1, n, d, "f32", causal,
             seed=100 + 8 * i + 2 * j + int(causal))
    for i, n in enumerate((64, 256, 1024, 2048))
    for j, d in enumerate((32, 64))
    for causal in (False, True)
]


def torch_dtype(name: str):
    if name == "bf16":
        return torch.bfloat16
    if name == "f32":
        return torch.float32
    raise ValueError(f"unknown element type {name!r}")


def default_scale(d: int) -> float:
    """1/sqrt(d) rounded to float32 (returned as the Python float of that value)."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32).item())


def make_qkv(B: int, H: int, N: int, d: int, dtype: str, seed: int,
             sigma_qk: float = 1.0, sigma_v: float = 1.0):
    """Q, K, V on the CPU, contiguous [B, H, N, d], in the given element type."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32) * sigma_qk
    k = torch.randn(shape, generator=g, dtype=torch.float32) * sigma_qk
    v = torch.randn(shape, generator=g, dtype=torch.float32) * sigma_v
    t = torch_dtype(dtype)
    return q.to(t).contiguous(), k.to(t).contiguous(), v.to(t).contiguous()


def make_qkv_cross(B: int, H: int, Nq: int, Nk: int, d: int, dtype: str, seed: int,
                   sigma_qk: float = 1.0, sigma_v: float = 1.0):
    """Q [B, H, Nq, d] and K, V [B, H, Nk, d] on the CPU, contiguous, in the given element
    type: Q, then K, then V drawn as N(0, 1) fp32 and scaled, as in ``make_qkv``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((B, H, Nq, d), generator=g, dtype=torch.float32) * sigma_qk
    k = torch.randn((B, H, Nk, d), generator=g, dtype=torch.float32) * sigma_qk
    v = torch.randn((B, H, Nk, d), generator=g, dtype=torch.float32) * sigma_v
    t = torch_dtype(dtype)
    return q.to(t).contiguous(), k.to(t).contiguous(), v.to(t).contiguous()


def sample_rows(N: int, count: int, seed: int):
    """Sorted distinct query rows for sampled checks: first, last, and seeded others."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 1000)
    picks = {0, N - 1, N // 2}
    if count > len(picks):
        extra = torch.randperm(N, generator=g)[: count].tolist()
        for r in extra:
            if len(picks) >= count:
                break
            picks.add(int(r))
    return sorted(picks)
