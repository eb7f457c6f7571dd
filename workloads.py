"""Seeded synthetic inputs for the attention workloads.

This module only draws random tensors; it holds none of the attention
arithmetic. Both the oracle-side tests and the HIP-side tests/bench take their
inputs from here, so the two sides see exactly the same values.

Recipe (one rule for every workload): a CPU ``torch.Generator`` seeded with
``seed`` draws Q, K, V and dO, in that order, as float32 standard normals of
the full ``[batch, heads, seq, head_dim]`` shape. Q is multiplied by
``q_std`` (the cross-attention workload uses sigma = 4, i.e. variance 16, to
stress the running-max rescale). bf16 workloads then cast each tensor with
round-to-nearest-even (``Tensor.to(torch.bfloat16)``). The teaching script of
page 1 ("05_flash_attention.py", section 2, demo_forward) draws its single
head the same way: seed 0, Q, K, V = randn in order, n = 100, d = 32.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    n_q: int
    n_k: int
    d: int
    dtype: str          # "bf16" or "f32"
    causal: bool | str  # False, True (top-left mask) or "bottom_right"
    q_std: float = 1.0

    def shape_q(self):
        return (self.batch, self.heads, self.n_q, self.d)

    def shape_k(self):
        return (self.batch, self.heads, self.n_k, self.d)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def fwd_flop(self) -> float:
        """4 * d FLOP per visible (query, key) pair and (batch, head): 4 n_q
        n_k d unmasked; halved for a causal mask over a square problem (the
        usual convention); the exact visible-pair count for a causal mask
        with n_q != n_k."""
        per_pair = 4.0 * self.d * self.batch * self.heads
        if not self.causal:
            return per_pair * self.n_q * self.n_k
        if self.n_q == self.n_k:
            return per_pair * self.n_q * self.n_k * 0.5
        off = self.n_k - self.n_q if self.causal == "bottom_right" else 0
        visible = sum(min(max(i + off + 1, 0), self.n_k) for i in range(self.n_q))
        return per_pair * visible

    def fwd_bwd_flop(self) -> float:
        """Backward counted as 2.5x forward, so fwd+bwd is 3.5x forward."""
        return 3.5 * self.fwd_flop()

    def with_causal(self, causal: bool) -> "Workload":
        return Workload(self.name, self.batch, self.heads, self.n_q, self.n_k,
                        self.d, self.dtype, causal, self.q_std)


# The five workloads. The first is the oracle-sized single head (n not a
# multiple of any tile); the third is the headline shape.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 1, 100, 100, 32, "f32", False),
    "tiny_f32_causal": Workload("tiny_f32_causal", 1, 1, 100, 100, 32, "f32", True),
    "self_b4h16_n1024_d64": Workload("self_b4h16_n1024_d64", 4, 16, 1024, 1024, 64, "bf16", False),
    "self_b2h32_n4096_d128_causal": Workload("self_b2h32_n4096_d128_causal", 2, 32, 4096, 4096, 128, "bf16", True),
    "long_b1h8_n32768_d128_causal": Workload("long_b1h8_n32768_d128_causal", 1, 8, 32768, 32768, 128, "bf16", True),
    "cross_b8h12_q1000_k3000_d64": Workload("cross_b8h12_q1000_k3000_d64", 8, 12, 1000, 3000, 64, "bf16", False, 4.0),
}

HEADLINE = "self_b2h32_n4096_d128_causal"


def make_inputs(w: Workload, seed: int = 0):
    """Return CPU tensors (Q, K, V, dO) in the workload's dtype."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q = torch.randn(w.shape_q(), generator=g, dtype=torch.float32)
    k = torch.randn(w.shape_k(), generator=g, dtype=torch.float32)
    v = torch.randn(w.shape_k(), generator=g, dtype=torch.float32)
    do = torch.randn(w.shape_q(), generator=g, dtype=torch.float32)
    if w.q_std != 1.0:
        q = q * w.q_std
    dt = w.torch_dtype
    return q.to(dt), k.to(dt), v.to(dt), do.to(dt)


def custom(batch, heads, n_q, n_k, d, dtype="bf16", causal=False, q_std=1.0, name="custom") -> Workload:
    return Workload(name, batch, heads, n_q, n_k, d, dtype, causal, q_std)
