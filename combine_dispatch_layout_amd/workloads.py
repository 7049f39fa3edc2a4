"""Seeded synthetic workloads for MoE token dispatch / combine.

This module only draws inputs: hidden rows, router top-k ids and router
weights.  It holds none of the dispatch/combine arithmetic, so both the HIP
path and the CPU oracle can take their inputs from it.

Shapes follow the expert-parallel rank shares the dispatcher pages are built
around (DeepSeek-V3-sized prefill and decode with 256 experts split over 8
ranks, plus a small parity case and a skewed long prefill):

  tiny          T=64,    H=256,  E=8,   L=8,   k=2, uniform distinct ids
  dsv3_prefill  T=4096,  H=7168, E=256, L=32,  k=8, uniform distinct ids
  ll_decode     T=128,   H=7168, E=256, L=32,  k=8, uniform, capacity 128*8
  fp8_dispatch  T=4096,  H=7168, E=256, L=32,  k=8, uniform (fp8 on scatter)
  zipf_prefill  T=16384, H=4096, E=128, L=128, k=8, Zipf(s=1.2) experts

Recipe (CPU ``torch.Generator``; seeds ``seed_base + {0: hidden, 1: ids,
2: logits}``):
  * hidden  = randn(T, H, float32) rounded to bfloat16;
  * ids     = multinomial(p, k, replacement=False) per token, p uniform over
              the E experts, or p_e ~ (e+1)^-s for the Zipf case (expert 0
              hottest); ids are global, the rank owns [expert_begin,
              expert_begin + L) and every other id is invalid for it;
  * weights = softmax over the k chosen slots of randn(T, k) logits (fp32).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    L: int
    k: int
    mode: str = "normal"          # "normal" | "ll" | "fp8"
    dist: str = "uniform"         # "uniform" | "zipf"
    zipf_s: float = 1.2
    expert_begin: int = 0
    cap: Optional[int] = None     # low-latency capacity per local expert
    num_ranks: int = 1            # EP ranks (for the expected_m hint)
    seed_base: int = 0

    def scaled(self, **kw) -> "Workload":
        """A copy with some sizes replaced (parity tests shrink T or H)."""
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", T=64, H=256, E=8, L=8, k=2, seed_base=1000),
    "dsv3_prefill": Workload("dsv3_prefill", T=4096, H=7168, E=256, L=32, k=8,
                             num_ranks=8, seed_base=2000),
    "ll_decode": Workload("ll_decode", T=128, H=7168, E=256, L=32, k=8,
                          mode="ll", cap=128 * 8, num_ranks=8, seed_base=3000),
    "fp8_dispatch": Workload("fp8_dispatch", T=4096, H=7168, E=256, L=32, k=8,
                             mode="fp8", num_ranks=8, seed_base=4000),
    "zipf_prefill": Workload("zipf_prefill", T=16384, H=4096, E=128, L=128,
                             k=8, dist="zipf", seed_base=5000),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def make_hidden(w: Workload) -> torch.Tensor:
    """[T, H] bfloat16 on the CPU, N(0, 1) rounded from float32."""
    g = _gen(w.seed_base + 0)
    return torch.randn(w.T, w.H, generator=g, dtype=torch.float32).to(torch.bfloat16)


def expert_probs(w: Workload) -> torch.Tensor:
    if w.dist == "uniform":
        return torch.ones(w.E, dtype=torch.float64)
    if w.dist == "zipf":
        r = torch.arange(1, w.E + 1, dtype=torch.float64)
        return r.pow(-w.zipf_s)
    raise ValueError("unknown expert distribution %r" % (w.dist,))


def make_topk_ids(w: Workload) -> torch.Tensor:
    """[T, k] int32 global expert ids, k distinct ids per token."""
    g = _gen(w.seed_base + 1)
    if w.T == 0:
        return torch.zeros(0, w.k, dtype=torch.int32)
    p = expert_probs(w).to(torch.float32).expand(w.T, w.E)
    return torch.multinomial(p, w.k, replacement=False, generator=g).to(torch.int32)


def make_topk_weights(w: Workload) -> torch.Tensor:
    """[T, k] float32 router weights: softmax of N(0,1) logits over k."""
    g = _gen(w.seed_base + 2)
    return torch.randn(w.T, w.k, generator=g, dtype=torch.float32).softmax(-1)


def make_inputs(w: Workload):
    """(hidden bf16 [T,H], topk_ids int32 [T,k], topk_weights f32 [T,k])."""
    return make_hidden(w), make_topk_ids(w), make_topk_weights(w)


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """The uint16 bit patterns of a CPU bfloat16 tensor (a view, no rounding)."""
    return x.contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_bf16(b: np.ndarray) -> torch.Tensor:
    """A CPU bfloat16 tensor holding the given uint16 bit patterns."""
    return torch.from_numpy(np.ascontiguousarray(b, np.uint16).view(np.int16)).view(
        torch.bfloat16)
