"""Seeded synthetic workloads: the only module both the library's tests and the
CPU oracle's tests draw inputs from.  It holds input generation only -- no step
of layout, dispatch, FP8 quantisation or combine.

The pages run their tests on real multi-GPU groups with random routing and
random activations; no dataset is involved.  These generators stand in for
them with the shapes and distributions of the five named workloads:

  tiny    128 tokens (4 sources x 32), hidden 256, 16 experts on 4 ranks, top-4
  normal  4096 tokens (8 sources x 512), hidden 7168, 256 experts on 8 ranks,
          top-8, 24 channels
  ll      32 source ranks x 128 tokens, hidden 7168, 256 experts on 32 ranks,
          top-8, seen from rank 0 (8 local experts)
  skewed  as normal, but experts drawn Zipf(1.2) over a random expert
          permutation, and exactly 10% of the top-k entries masked to -1
  large   16384 tokens (64 sources x 256), hidden 7168, 256 experts on 64
          ranks (8 RDMA groups of 8), top-8, FP8-cast dispatch

All draws come from one ``torch.Generator`` seeded per call, in a fixed order
(routing, then weights, then activations), so every consumer sees identical
bytes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class NormalWorkload:
    name: str
    S: int            # logical source partitions
    T: int            # tokens per source partition
    H: int            # hidden size
    E: int            # experts
    R: int            # logical ranks
    K: int            # top-k
    C: int            # channels
    expert_alignment: int = 1
    routing: str = "uniform"     # "uniform" | "zipf"
    zipf_s: float = 0.0
    mask_frac: float = 0.0
    x_kind: str = "bf16"         # "bf16" | "fp8" (pre-quantised) | "bf16_cast_fp8"

    @property
    def N(self) -> int:
        return self.S * self.T

    @property
    def L(self) -> int:
        return self.E // self.R


@dataclass(frozen=True)
class LLWorkload:
    name: str
    S: int            # source ranks (= R)
    T: int            # tokens per source rank
    M: int            # max dispatch tokens per rank (slot capacity per (expert, source))
    H: int
    E: int
    R: int
    K: int
    dest_rank: int

    @property
    def N(self) -> int:
        return self.S * self.T

    @property
    def L(self) -> int:
        return self.E // self.R


TINY = NormalWorkload("tiny", S=4, T=32, H=256, E=16, R=4, K=4, C=24)
NORMAL = NormalWorkload("normal", S=8, T=512, H=7168, E=256, R=8, K=8, C=24)
LL = LLWorkload("ll", S=32, T=128, M=128, H=7168, E=256, R=32, K=8, dest_rank=0)
SKEWED = NormalWorkload("skewed", S=8, T=512, H=7168, E=256, R=8, K=8, C=24, routing="zipf", zipf_s=1.2,
                        mask_frac=0.1)
LARGE = NormalWorkload("large", S=64, T=256, H=7168, E=256, R=64, K=8, C=24, x_kind="bf16_cast_fp8")

WORKLOADS = {w.name: w for w in (TINY, NORMAL, LL, SKEWED, LARGE)}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def topk_uniform(N: int, E: int, K: int, g: torch.Generator) -> torch.Tensor:
    """K distinct experts per token, uniform: the top-K of E i.i.d. U(0,1) scores."""
    if N == 0:
        return torch.empty((0, K), dtype=torch.int64)
    scores = torch.rand((N, E), generator=g)
    return scores.topk(K, dim=1).indices.to(torch.int64).contiguous()


def topk_zipf(N: int, E: int, K: int, s: float, mask_frac: float, g: torch.Generator) -> torch.Tensor:
    """K distinct experts per token drawn without replacement from p_i ~ i^-s
    (i = 1..E) placed on a random permutation of the experts (Gumbel-top-k);
    then exactly floor(mask_frac * N * K) entries, chosen uniformly, set to -1."""
    perm = torch.randperm(E, generator=g)
    logp = torch.empty(E, dtype=torch.float64)
    logp[perm] = -s * torch.log(torch.arange(1, E + 1, dtype=torch.float64))
    u = torch.rand((N, E), generator=g, dtype=torch.float64).clamp_min(1e-300)
    gumbel = -torch.log(-torch.log(u))
    idx = (logp.unsqueeze(0) + gumbel).topk(K, dim=1).indices.to(torch.int64)
    n_mask = int(math.floor(mask_frac * N * K))
    if n_mask > 0:
        flat = idx.reshape(-1)
        pick = torch.randperm(N * K, generator=g)[:n_mask]
        flat[pick] = -1
        idx = flat.reshape(N, K)
    return idx.contiguous()


def gate_weights(N: int, K: int, g: torch.Generator) -> torch.Tensor:
    """topk_weights = softmax over k of N(0,1) logits, fp32."""
    return torch.softmax(torch.randn((N, K), generator=g, dtype=torch.float32), dim=1).contiguous()


def activations(N: int, H: int, g: torch.Generator) -> torch.Tensor:
    """bf16 activations: N(0,1) fp32 rounded to bf16."""
    return torch.randn((N, H), generator=g, dtype=torch.float32).to(torch.bfloat16).contiguous()


def normal_inputs(w: NormalWorkload, seed: int = 0) -> dict:
    """x [N][H] bf16, topk_idx [N][K] int64, topk_weights [N][K] fp32 (CPU tensors)."""
    g = _gen(seed)
    if w.routing == "uniform":
        idx = topk_uniform(w.N, w.E, w.K, g)
    elif w.routing == "zipf":
        idx = topk_zipf(w.N, w.E, w.K, w.zipf_s, w.mask_frac, g)
    else:
        raise ValueError(w.routing)
    wts = gate_weights(w.N, w.K, g)
    x = activations(w.N, w.H, g)
    return dict(x=x, topk_idx=idx, topk_weights=wts)


def ll_inputs(w: LLWorkload, seed: int = 0) -> dict:
    """x [S*T][H] bf16 and topk_idx [S*T][K] int64 for the low-latency workload."""
    g = _gen(seed)
    idx = topk_uniform(w.N, w.E, w.K, g)
    x = activations(w.N, w.H, g)
    return dict(x=x, topk_idx=idx)


def structured_x(S: int, T: int, H: int) -> torch.Tensor:
    """x whose row (s, t) names its own source token in exact bf16 integers:
    channel h holds s, t % 256 or t // 256 for h % 3 = 0, 1, 2 (all < 256,
    so exactly representable), for checking placements by eye."""
    s = torch.arange(S).repeat_interleave(T)
    t = torch.arange(T).repeat(S)
    cols = torch.stack([s, t % 256, t // 256], dim=1).to(torch.float32)   # [N, 3]
    return cols[:, torch.arange(H) % 3].to(torch.bfloat16).contiguous()


def expert_outputs(rows: int, H: int, seed: int = 1) -> torch.Tensor:
    """Synthetic expert outputs in the receive layout: bf16 N(0,1)."""
    return activations(rows, H, _gen(seed))


def bf16_bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (for the CPU oracle)."""
    return t.contiguous().view(torch.int16).numpy().view("uint16")
