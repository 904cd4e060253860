"""Capacity planning for a batch of decode sequences on one GPU (host
arithmetic only; nothing here touches the GPU).

(P1, P2, P3: the three pages listed, with their titles, at the top of
include/qkdec.h.)

* P1 "Where it stops, and the argument I got wrong in May": the KV cache is
  given a fixed fraction (0.85) of device memory minus the weights; that
  budget divided by the bytes one token costs across all layers is the number
  of tokens the card holds, and split over the batch it is the context each
  sequence can keep.
* P2 "The two halves of a decode-step memory bill" and "Where the private read
  overtakes the shared one": a step reads the shared weights W once plus every
  sequence's own cache, W + sum_b L_b k bytes.  B sequences at context L
  therefore run B (W + L k) / (W + B L k) times faster in aggregate than one,
  and the private read equals the shared one at L* = W / (B k).
* P2 "What a long-running swarm should actually tune": the live batch size
  times each sequence's context is the step's KV traffic.
* P3 "What the sagging ceiling costs in tokens per second": with the step
  bound by memory bandwidth, the aggregate rate is B / ((W + B L k) / BW).

Byte counts follow the library's storage formats (include/qkdec.h): fp16 2
bytes per element, Q8_0 34 bytes per 32 elements, E4M3 1 byte; a cache
capacity is a multiple of 32 tokens.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Iterable

VRAM_FRACTION = 0.85

# bytes per cached element of (keys, values) for each cache kind
_ELEMENT_BYTES = {
    "f16": (2.0, 2.0),
    "q8_0": (34 / 32, 34 / 32),
    "q8k_f16v": (34 / 32, 2.0),
    "f16k_q8v": (2.0, 34 / 32),
    "fp8": (1.0, 1.0),
}

Q4K_BLOCK_BYTES = 144   # 256 weights


def kv_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int, kind: str) -> float:
    """Bytes one cached token costs across all layers, keys and values."""
    if kind not in _ELEMENT_BYTES:
        raise ValueError(f"unknown cache kind {kind!r}")
    kb, vb = _ELEMENT_BYTES[kind]
    return n_layers * n_kv_heads * head_dim * (kb + vb)


def model_weight_bytes(n_layers: int, hidden: int, n_q_heads: int, n_kv_heads: int, head_dim: int, ffn: int,
                       vocab: int) -> int:
    """Bytes a step reads once for the whole batch: the Q4_K projections of
    every layer (QKV, O, gate/up, down), the fp16 LM head and the fp32 norm
    gains (two per layer and the final one).  The embedding rows gathered per
    token are not counted."""
    def q4k(n, k):
        if k % 256:
            raise ValueError("Q4_K rows need K % 256 == 0")
        return n * (k // 256) * Q4K_BLOCK_BYTES
    qkv = (n_q_heads + 2 * n_kv_heads) * head_dim
    layer = q4k(qkv, hidden) + q4k(hidden, n_q_heads * head_dim) + q4k(2 * ffn, hidden) + q4k(hidden, ffn)
    return n_layers * layer + vocab * hidden * 2 + (2 * n_layers + 1) * hidden * 4


def step_bytes(weight_bytes: float, lengths: Iterable[float], k: float) -> float:
    """W + sum_b L_b k: the bytes one decode step reads."""
    return weight_bytes + kv_traffic_bytes(lengths, k)


def kv_traffic_bytes(lengths: Iterable[float], k: float) -> float:
    """The private part of a step's reads: sum over live sequences of context x k."""
    return sum(float(n) for n in lengths) * k


def speedup(batch: int, context: float, weight_bytes: float, k: float) -> float:
    """Aggregate rate of `batch` sequences at `context` over one sequence, for a
    bandwidth-bound step."""
    return batch * (weight_bytes + context * k) / (weight_bytes + batch * context * k)


def crossover_context(weight_bytes: float, batch: int, k: float) -> float:
    """Context per sequence at which the batch's KV reads equal the weight read."""
    return weight_bytes / (batch * k)


def ceiling_tok_s(bandwidth: float, weight_bytes: float, batch: int, context: float, k: float) -> float:
    """Aggregate tokens/s of a step bound by `bandwidth` bytes/s."""
    return batch * bandwidth / (weight_bytes + batch * context * k)


def slot_capacity(context: int, steps: int) -> int:
    """Smallest cache capacity (a multiple of 32) for a sequence that starts at
    `context` cached tokens and decodes `steps` more."""
    need = context + steps
    return max(32, (need + 31) // 32 * 32)


@dataclass(frozen=True)
class CapacityPlan:
    vram_bytes: float
    weight_bytes: float
    kv_bytes_per_token: float
    fraction: float = VRAM_FRACTION

    @property
    def budget_bytes(self) -> float:
        """fraction x VRAM - W (negative when the weights alone do not fit)."""
        return self.fraction * self.vram_bytes - self.weight_bytes

    @property
    def total_tokens(self) -> int:
        """Cached tokens the budget holds over all sequences."""
        return max(0, math.floor(self.budget_bytes / self.kv_bytes_per_token))

    def context_per_sequence(self, batch: int) -> int:
        """Context each of `batch` equal sequences can hold."""
        if batch < 1:
            raise ValueError("batch must be >= 1")
        return self.total_tokens // batch

    def max_batch(self, context: int) -> int:
        """Most sequences of `context` tokens the budget holds."""
        if context < 1:
            raise ValueError("context must be >= 1")
        return self.total_tokens // context

    def fits(self, lengths: Iterable[int]) -> bool:
        """Whether sequences of these lengths fit the budget together."""
        return sum(int(n) for n in lengths) <= self.total_tokens


def plan_capacity(vram_bytes: float, weight_bytes: float, kv_bytes_per_token_: float,
                  fraction: float = VRAM_FRACTION) -> CapacityPlan:
    if not (0.0 < fraction <= 1.0):
        raise ValueError("fraction must be in (0, 1]")
    if kv_bytes_per_token_ <= 0:
        raise ValueError("kv_bytes_per_token must be positive")
    return CapacityPlan(float(vram_bytes), float(weight_bytes), float(kv_bytes_per_token_), fraction)
