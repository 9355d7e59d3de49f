"""Seeded synthetic inputs and the named workloads.

This module only draws random numbers and describes shapes; it holds none
of the attention arithmetic.  Both the HIP path and the oracle read the
identical bf16 tensors it returns.

Recipe: one CPU torch.Generator seeded with `seed`; Q, then K, then V are
drawn in float32 with the stated distribution and rounded to bfloat16
(round-to-nearest-even, torch's conversion).
  "normal":  randn * sigma
  "uniform": rand * 2 - 1      (U(-1, 1))
Layouts: q [batch, T, n_h, hd], k and v [batch, s_k, n_kv_h, hd], head dim
contiguous.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_h: int
    n_kv_h: int
    T: int
    s_k: int
    hd: int
    causal: bool = False
    window: int = 0
    q_dist: str = "normal"
    k_dist: str = "normal"
    v_dist: str = "normal"
    sigma: float = 1.0
    split_len: Optional[int] = None  # set: decode through split-KV partitions + LSE merge
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.hd)

    @property
    def n_split(self) -> int:
        return 1 if self.split_len is None else -(-self.s_k // self.split_len)


def _draw(g: torch.Generator, shape, dist: str, sigma: float) -> torch.Tensor:
    dev = g.device
    if dist == "normal":
        x = torch.randn(shape, generator=g, dtype=torch.float32, device=dev) * sigma
    elif dist == "uniform":
        x = torch.rand(shape, generator=g, dtype=torch.float32, device=dev) * 2.0 - 1.0
    else:
        raise ValueError(dist)
    return x.to(torch.bfloat16)


def make_qkv(w: Workload, seed: Optional[int] = None, device: str = "cpu"):
    """Returns (q, k, v) as bf16 tensors for workload w.

    device="cpu" draws with the CPU generator (the recipe above).  For the
    gigabyte-sized workloads device="cuda" draws with the seeded device
    generator instead (same recipe, a different random stream); whoever
    checks the result copies those exact bf16 tensors to the host."""
    g = torch.Generator(device=device)
    g.manual_seed(w.seed if seed is None else seed)
    q = _draw(g, (w.batch, w.T, w.n_h, w.hd), w.q_dist, w.sigma)
    k = _draw(g, (w.batch, w.s_k, w.n_kv_h, w.hd), w.k_dist, w.sigma)
    v = _draw(g, (w.batch, w.s_k, w.n_kv_h, w.hd), w.v_dist, w.sigma)
    return q, k, v


def randn_bf16(shape, seed: int, sigma: float = 1.0) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return _draw(g, shape, "normal", sigma)


def rand_f32(shape, seed: int, lo: float = -1.0, hi: float = 1.0) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.rand(shape, generator=g, dtype=torch.float32) * (hi - lo) + lo


# ---------------------------------------------------------------------------
# The five workloads of the target (all seed 0).
# ---------------------------------------------------------------------------

SINGLE_HEAD_DECODE = Workload("decode_b1_h1_sk128_hd64", 1, 1, 1, 1, 128, 64)


def mqa_decode(hd: int, s_k: int) -> Workload:
    """128 query heads sharing one KV head, batch 8, T = 1."""
    return Workload(f"mqa_decode_b8_h128_hd{hd}_sk{s_k}", 8, 128, 1, 1, s_k, hd)


MQA_DECODE_GRID: List[Workload] = [mqa_decode(hd, sk) for hd in (64, 128, 256, 512)
                                   for sk in (128, 256, 384, 512)]

GQA_SPLITKV_DECODE = Workload("gqa_splitkv_decode_b32_h64_kv8_sk8192_hd128", 32, 64, 8, 1, 8192, 128,
                              v_dist="uniform", split_len=128)


def mha_causal_prefill(T: int, s_k: int, hd: int) -> Workload:
    """MHA, batch 4, 32 heads, queries at the last T positions, causal."""
    return Workload(f"mha_causal_prefill_b4_h32_T{T}_sk{s_k}_hd{hd}", 4, 32, 32, T, s_k, hd, causal=True)


MHA_PREFILL_GRID: List[Workload] = [mha_causal_prefill(T, sk, hd) for T in (1, 4, 32, 128)
                                    for sk in (128, 256, 384, 512) for hd in (64, 128, 256, 512)]

SWA_MQA_PREFILL = Workload("swa_mqa_prefill_b2_h16_T128_sk4096_hd512_w128", 2, 16, 1, 128, 4096, 512,
                           causal=True, window=128, sigma=0.5)

ALL_WORKLOADS: List[Workload] = ([SINGLE_HEAD_DECODE] + MQA_DECODE_GRID + [GQA_SPLITKV_DECODE]
                                 + MHA_PREFILL_GRID + [SWA_MQA_PREFILL])

# ---------------------------------------------------------------------------
# Beyond the five: long prefill (T up to s_k, full causal), where the
# arithmetic intensity passes the MFMA ridge.
# ---------------------------------------------------------------------------


def gqa_causal_prefill_long(T: int, hd: int, batch: int = 2, n_h: int = 32, n_kv_h: int = 8) -> Workload:
    """GQA (group 4), a whole causal prompt: T = s_k."""
    return Workload(f"gqa_causal_prefill_long_b{batch}_h{n_h}_kv{n_kv_h}_T{T}_sk{T}_hd{hd}", batch, n_h, n_kv_h,
                    T, T, hd, causal=True)


LONG_PREFILL = gqa_causal_prefill_long(4096, 128)

# One GPU's share of the GQA split-KV decode workload sharded over 8 GPUs:
# by KV head (one KV head and its 8 query heads per GPU), or by sequence
# (1024 of the 8192 keys per GPU, its 8 partitions written into its slots of
# a 64-slot partial buffer that is exchanged and merged once).
HEAD_SHARD_DECODE = Workload("gqa_splitkv_decode_head_shard_b32_h8_kv1_sk8192_hd128", 32, 8, 1, 1, 8192, 128,
                             v_dist="uniform", split_len=128)
SEQ_SHARD_DECODE = Workload("gqa_splitkv_decode_seq_shard_b32_h64_kv8_sk1024_hd128", 32, 64, 8, 1, 1024, 128,
                            v_dist="uniform", split_len=128)
SHARDS = 8

# A ragged decode batch: the GQA split-KV workload's shapes with per-row key
# counts drawn uniformly from 1..s_k (the cache holds s_k per row).
RAGGED_DECODE = Workload("gqa_ragged_decode_b32_h64_kv8_skmax8192_hd128", 32, 64, 8, 1, 8192, 128,
                         v_dist="uniform", split_len=128)


def ragged_lengths(batch: int, s_max: int, seed: int = 0) -> torch.Tensor:
    """int32 [batch] key counts, uniform on 1..s_max (CPU generator)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randint(1, s_max + 1, (batch,), generator=g, dtype=torch.int32)
