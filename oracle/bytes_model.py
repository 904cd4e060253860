"""The pages' byte model of a batched decode step (oracle; test infrastructure only).
(P1, P2, P3: the three pages listed, with their titles, in oracle/__init__.py.)

P2 "The two halves of a decode-step memory bill": with B sequences each
holding L cached tokens, a step moves the shared weights W once plus the
private KV bytes B*L*k, where k is the KV cost of one token; per generated
token that is W/B + L*k.
P2 "Where the private read overtakes the shared one": the B-sequence speedup
over running them one at a time is B*(W + L*k) / (W + B*L*k), and the private
read equals the shared one at L* = W / (B*k).
P1 "Where it stops, and the argument I got wrong in May": the KV budget is
0.85 of device memory minus the weights, divided by the per-token cost.
P3 "The crossover is just a byte count" (chart caption): the fitted step time
t(B, C) = 16.9 + B*(1.1 + k*C) ms.
"""
from __future__ import annotations

Q4K_BLOCK_BYTES = 144
QK_K = 256


def q4k_matrix_bytes(n_rows: int, n_cols: int) -> int:
    return n_rows * (n_cols // QK_K) * Q4K_BLOCK_BYTES


def layer_weight_bytes(dims) -> int:
    hq = dims.n_q_heads * dims.head_dim
    return (q4k_matrix_bytes(dims.qkv_rows, dims.hidden) + q4k_matrix_bytes(dims.hidden, hq)
            + q4k_matrix_bytes(2 * dims.ffn, dims.hidden) + q4k_matrix_bytes(dims.hidden, dims.ffn))


def weight_bytes(dims) -> int:
    """Shared bytes read once per step: Q4_K layers, fp16 LM head, fp32 norm gains.

    The embedding gather reads only B rows and is not part of W.
    """
    q4k = dims.n_layers * layer_weight_bytes(dims)
    lm_head = dims.vocab * dims.hidden * 2
    norms = (2 * dims.n_layers + 1) * dims.hidden * 4
    return q4k + lm_head + norms


def kv_bytes_per_token(dims, kind: str) -> float:
    """Bytes one cached token costs across all layers, K and V.

    fp16: 2 bytes per element.  Q8_0: 34 bytes per 32 elements (32 int8 + one
    fp16 scale); the pages round this to one byte per element.  fp8: one byte
    per element, no scale (half of fp16, P2 "What a long-running swarm should
    actually tune").
    """
    elems = dims.n_layers * dims.n_kv_heads * dims.head_dim * 2
    if kind == "f16":
        return elems * 2
    if kind == "q8_0":
        return elems * 34 // 32
    if kind == "fp8":
        return elems
    raise ValueError(kind)


def step_bytes(w: float, lengths, k: float) -> float:
    """W + sum_b L_b * k."""
    return w + sum(lengths) * k


def bytes_per_token(w: float, batch: int, length: float, k: float) -> float:
    return w / batch + length * k


def speedup(batch: int, length: float, w: float, k: float) -> float:
    return batch * (w + length * k) / (w + batch * length * k)


def crossover(w: float, batch: int, k: float) -> float:
    return w / (batch * k)


def kv_capacity_tokens(vram: float, w: float, k: float, frac: float = 0.85) -> float:
    return (frac * vram - w) / k


def kv_budget_bytes(vram: float, w: float, frac: float = 0.85) -> float:
    return frac * vram - w


def fitted_step_ms(batch: int, context: float, k_ms_per_token: float,
                   base_ms: float = 16.9, per_seq_ms: float = 1.1) -> float:
    return base_ms + batch * (per_seq_ms + k_ms_per_token * context)
