"""Seeded synthetic inputs for the attention forward workloads.

This module only draws random tensors; it contains none of the attention
arithmetic, so both the HIP path and the CPU oracle can consume its output.

Recipe (per workload k, 1-based): ``torch.Generator('cpu').manual_seed(1000 + k)``;
Q, K, V are drawn in that order in float32 on the CPU, any row scaling is applied in
float32, then each tensor is cast to the workload's 16-bit type with
round-to-nearest-even. The same 16-bit tensors, upcast losslessly, feed the oracle.

Shapes and distributions follow the pages' own examples: the blog's single-head
[128, 64] walk-through (64x64 tiles), ch. 14's N = 4096, d = 64 traffic example,
and the remaining mixes of length, head size, causality, ragged tails and
large running-maximum jumps that exercise the online-softmax rescaling.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    index: int                 # 1-based; seed = 1000 + index
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str                 # "f16" | "bf16"
    causal: bool
    scale: float
    qk_std: float = 1.0        # Q and K ~ N(0, qk_std^2)
    v_dist: str = "normal"     # "normal" (N(0, v_std^2)) | "uniform" (U(-1, 1))
    v_std: float = 1.0
    spike_frac: float = 0.0    # fraction of Q rows per (b, h) multiplied by spike_mult
    spike_mult: float = 1.0
    tile: tuple | None = None  # forced (block_m, block_n), if the workload names one

    @property
    def torch_dtype(self):
        return torch.float16 if self.dtype == "f16" else torch.bfloat16

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def flops(self) -> float:
        """Counted FLOPs: 4 B H N^2 d, halved for causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def label(self) -> str:
        return (f"B{self.B}_H{self.H}_N{self.N}_d{self.d}_{self.dtype}"
                f"{'_causal' if self.causal else ''}")


WORKLOADS = {
    1: Workload(1, "single_head_128x64_f16", 1, 1, 128, 64, "f16", False, 1 / 8, tile=(64, 64)),
    2: Workload(2, "n4096_d64_f16", 2, 16, 4096, 64, "f16", False, 1 / 8),
    3: Workload(3, "n2048_d128_bf16_causal", 4, 32, 2048, 128, "bf16", True, 1 / math.sqrt(128)),
    4: Workload(4, "n16384_d128_bf16_spiked", 1, 16, 16384, 128, "bf16", False, 1 / math.sqrt(128),
                v_dist="uniform", spike_frac=0.01, spike_mult=20.0),
    5: Workload(5, "n1000_d64_f16_causal_ragged", 8, 16, 1000, 64, "f16", True, 1 / 8,
                qk_std=0.5, v_std=0.5),
}


@dataclass(frozen=True)
class GeneralWorkload:
    """A workload of the general and split-KV entry points: Hq query heads over Hk K/V
    heads, Nq queries against Nk keys (causal = bottom-right alignment)."""
    index: int                 # seed = 1000 + index
    name: str
    B: int
    Hq: int
    Hk: int
    Nq: int
    Nk: int
    d: int
    dtype: str
    causal: bool
    scale: float
    v_std: float = 1.0

    @property
    def torch_dtype(self):
        return torch.float16 if self.dtype == "f16" else torch.bfloat16

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def visible_pairs(self) -> int:
        """(query, key) pairs the mask leaves visible, per (batch, head)."""
        if not self.causal:
            return self.Nq * self.Nk
        off = self.Nk - self.Nq
        return sum(max(0, min(self.Nk, i + off + 1)) for i in range(self.Nq))

    @property
    def flops(self) -> float:
        """4 d FLOPs per visible (query, key) pair and head (both products)."""
        return 4.0 * self.d * self.B * self.Hq * self.visible_pairs

    @property
    def hbm_bytes(self) -> int:
        """Compulsory traffic: Q, K, V read once, O and LSE written once."""
        e = 2
        return (2 * self.B * self.Hq * self.Nq * self.d * e + 2 * self.B * self.Hk * self.Nk * self.d * e
                + 4 * self.B * self.Hq * self.Nq)


# Split-KV workloads: long-context decoding (one new query row per head against a
# 128K-key cache, grouped K/V heads: ch. 14 §14.7.1's case), and one GPU's share of
# the N = 16384 workload when its 16 heads are divided over 8 GPUs (2 heads each).
SPLIT_WORKLOADS = {
    6: GeneralWorkload(6, "decode_nk131072_hq32_hk8_d128_bf16", 1, 32, 8, 1, 131072, 128, "bf16", True,
                       1 / math.sqrt(128)),
    7: GeneralWorkload(7, "n16384_d128_bf16_h2_shard", 1, 2, 2, 16384, 16384, 128, "bf16", False,
                       1 / math.sqrt(128)),
}


def make_general_inputs(w: GeneralWorkload):
    """(q, k, v) CPU tensors: q [B, Hq, Nq, d], k and v [B, Hk, Nk, d]; Q, K ~ N(0, 1),
    V ~ N(0, v_std^2), drawn in that order in float32 and rounded to the 16-bit type."""
    g = torch.Generator("cpu").manual_seed(w.seed)
    q = torch.randn((w.B, w.Hq, w.Nq, w.d), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, w.Hk, w.Nk, w.d), generator=g, dtype=torch.float32)
    v = torch.randn((w.B, w.Hk, w.Nk, w.d), generator=g, dtype=torch.float32) * w.v_std
    dt = w.torch_dtype
    return q.to(dt), k.to(dt), v.to(dt)


def spike_count(w: Workload) -> int:
    return int(round(w.spike_frac * w.N))


def make_inputs(w: Workload, seed: int | None = None):
    """Return (q, k, v) CPU tensors [B, H, N, d] in the workload's 16-bit type, plus the
    spiked row indices per (b, h) as a [B, H, count] int64 tensor (empty if none)."""
    g = torch.Generator("cpu").manual_seed(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.N, w.d)
    q = torch.randn(shape, generator=g, dtype=torch.float32) * w.qk_std
    k = torch.randn(shape, generator=g, dtype=torch.float32) * w.qk_std
    if w.v_dist == "uniform":
        v = torch.rand(shape, generator=g, dtype=torch.float32) * 2.0 - 1.0
    else:
        v = torch.randn(shape, generator=g, dtype=torch.float32) * w.v_std
    cnt = spike_count(w)
    spikes = torch.empty((w.B, w.H, cnt), dtype=torch.int64)
    for b in range(w.B):
        for h in range(w.H):
            if cnt:
                idx = torch.randperm(w.N, generator=g)[:cnt]
                spikes[b, h] = idx
                q[b, h, idx] *= w.spike_mult
    dt = w.torch_dtype
    return q.to(dt), k.to(dt), v.to(dt), spikes


def make_random(B: int, H: int, N: int, d: int, dtype: str, seed: int, std: float = 1.0):
    """Plain N(0, std^2) Q, K, V of any shape (for edge-case tests)."""
    g = torch.Generator("cpu").manual_seed(seed)
    dt = torch.float16 if dtype == "f16" else torch.bfloat16
    shape = (B, H, N, d)
    out = [torch.randn(shape, generator=g, dtype=torch.float32) * std for _ in range(3)]
    return tuple(t.to(dt) for t in out)
