"""Seeded synthetic inputs shared by the tests, the oracle's callers and bench.py.

This module draws random numbers and lays them into the storage formats; it
computes nothing that the decode step computes (no dequantization, no matmul,
no attention).  Both the HIP path and the oracle consume exactly the arrays
produced here.

Distributions (the workloads of the batched-decode pages, with Qwen-shaped
synthetic weights standing in for a trained model):

* Q4_K super-block: fp16 ``d`` and ``dmin`` each |N(0,1)|*1e-3, the other 140
  bytes uniform random, so every 6-bit scale/min is uniform in 0..63 and every
  4-bit quant uniform in 0..15 (the packing is a bijection).
* fp16 tensors (embedding, hidden states, fp16 KV, q): N(0,1) rounded to fp16.
* LM head: N(0,1)/sqrt(hidden) in fp16, so logits are O(1).
* RMSNorm gains: 1 + 0.1*N(0,1) in fp32.
* Q8_0 KV: int8 uniform in -127..127, fp16 scale |N(0,1)|*0.02 per 32 values.

Seeds: a config uses ``numpy.random.SeedSequence(seed)``; every tensor gets its
own child stream from ``spawn`` in declaration order.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

Q4K_BLOCK_BYTES = 144
Q4K_WEIGHTS = 256
Q4K_ROW_TILE = 16
Q8_BLOCK = 32


@dataclass(frozen=True)
class ModelDims:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-6
    rope_base: float = 1e6

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


TOY = ModelDims(n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=64,
                ffn=1536, vocab=4096)
QWEN_SHAPED = ModelDims(n_layers=36, hidden=4096, n_q_heads=32, n_kv_heads=8,
                        head_dim=128, ffn=12288, vocab=151936)


class Streams:
    """Hands out one independent numpy Generator per tensor, in call order."""

    def __init__(self, seed: int):
        self._ss = np.random.SeedSequence(seed)

    def next(self) -> np.random.Generator:
        (child,) = self._ss.spawn(1)
        return np.random.Generator(np.random.PCG64(child))


def f16_normal(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x.astype(np.float16)


def q4k_matrix(rng: np.random.Generator, n_rows: int, n_cols: int) -> np.ndarray:
    """Random Q4_K matrix bytes in the row-tile-interleaved order.

    Returns uint8 [n_rows/16, n_cols/256, 16, 144]: tile of 16 rows, super-block
    column, row within the tile, block bytes.  Bytes 0-1 / 2-3 of every block are
    the fp16 ``d`` / ``dmin`` (little-endian); the other 140 bytes are uniform.
    """
    assert n_rows % Q4K_ROW_TILE == 0 and n_cols % Q4K_WEIGHTS == 0
    shape = (n_rows // Q4K_ROW_TILE, n_cols // Q4K_WEIGHTS, Q4K_ROW_TILE)
    blocks = rng.integers(0, 256, size=shape + (Q4K_BLOCK_BYTES,), dtype=np.uint8)
    d = np.abs(rng.standard_normal(size=shape + (2,))) * 1e-3
    blocks[..., 0:4] = d.astype(np.float16).view(np.uint8).reshape(shape + (4,))
    return blocks


def gains(rng: np.random.Generator, n: int) -> np.ndarray:
    return (1.0 + 0.1 * rng.standard_normal(size=n)).astype(np.float32)


@dataclass
class LayerWeights:
    w_qkv: np.ndarray       # Q4_K [qkv_rows x hidden], rows = [q heads; k heads; v heads]
    w_o: np.ndarray         # Q4_K [hidden x n_q_heads*head_dim]
    w_gate_up: np.ndarray   # Q4_K [2*ffn x hidden], rows = [gate; up]
    w_down: np.ndarray      # Q4_K [hidden x ffn]
    norm_attn: np.ndarray   # fp32 [hidden]
    norm_ffn: np.ndarray    # fp32 [hidden]


@dataclass
class ModelWeights:
    dims: ModelDims
    embed: np.ndarray       # fp16 [vocab x hidden]
    lm_head: np.ndarray     # fp16 [vocab x hidden]
    norm_final: np.ndarray  # fp32 [hidden]
    layers: List[LayerWeights] = field(default_factory=list)


def make_model(dims: ModelDims, seed: int, n_layers: Optional[int] = None) -> ModelWeights:
    """Synthetic model with the given shapes (``n_layers`` may cut the depth)."""
    st = Streams(seed)
    embed = f16_normal(st.next(), (dims.vocab, dims.hidden))
    lm_head = f16_normal(st.next(), (dims.vocab, dims.hidden), scale=1.0 / np.sqrt(dims.hidden))
    norm_final = gains(st.next(), dims.hidden)
    layers = []
    nl = dims.n_layers if n_layers is None else n_layers
    hq = dims.n_q_heads * dims.head_dim
    for _ in range(nl):
        layers.append(LayerWeights(
            w_qkv=q4k_matrix(st.next(), dims.qkv_rows, dims.hidden),
            w_o=q4k_matrix(st.next(), dims.hidden, hq),
            w_gate_up=q4k_matrix(st.next(), 2 * dims.ffn, dims.hidden),
            w_down=q4k_matrix(st.next(), dims.hidden, dims.ffn),
            norm_attn=gains(st.next(), dims.hidden),
            norm_ffn=gains(st.next(), dims.hidden),
        ))
    return ModelWeights(dims=dims, embed=embed, lm_head=lm_head, norm_final=norm_final, layers=layers)


@dataclass
class KVLayerF16:
    """Logical fp16 cache of one layer: k, v [n_slots, n_kv, capacity, head_dim]."""
    k: np.ndarray
    v: np.ndarray


@dataclass
class KVLayerQ8:
    """Logical Q8_0 cache of one layer.

    kq, vq: int8 [n_slots, n_kv, capacity, head_dim];
    ks, vs: fp16 [n_slots, n_kv, capacity, head_dim/32] (one scale per 32 values
    of one token and head).
    """
    kq: np.ndarray
    ks: np.ndarray
    vq: np.ndarray
    vs: np.ndarray


def kv_cache_f16(rng_k: np.random.Generator, rng_v: np.random.Generator, n_slots: int,
                 n_kv: int, capacity: int, head_dim: int, filled) -> KVLayerF16:
    """fp16 N(0,1) for positions < filled[slot], zero beyond."""
    shape = (n_slots, n_kv, capacity, head_dim)
    k = np.zeros(shape, np.float16)
    v = np.zeros(shape, np.float16)
    for s in range(n_slots):
        n = int(filled[s])
        k[s, :, :n] = f16_normal(rng_k, (n_kv, n, head_dim))
        v[s, :, :n] = f16_normal(rng_v, (n_kv, n, head_dim))
    return KVLayerF16(k=k, v=v)


def kv_cache_q8(rng_k: np.random.Generator, rng_v: np.random.Generator, n_slots: int,
                n_kv: int, capacity: int, head_dim: int, filled) -> KVLayerQ8:
    shape = (n_slots, n_kv, capacity, head_dim)
    sshape = (n_slots, n_kv, capacity, head_dim // Q8_BLOCK)
    out = KVLayerQ8(kq=np.zeros(shape, np.int8), ks=np.zeros(sshape, np.float16),
                    vq=np.zeros(shape, np.int8), vs=np.zeros(sshape, np.float16))
    for s in range(n_slots):
        n = int(filled[s])
        for rng, q, sc in ((rng_k, out.kq, out.ks), (rng_v, out.vq, out.vs)):
            q[s, :, :n] = rng.integers(-127, 128, size=(n_kv, n, head_dim), dtype=np.int8)
            sc[s, :, :n] = (np.abs(rng.standard_normal(size=(n_kv, n, head_dim // Q8_BLOCK)))
                            * 0.02).astype(np.float16)
    return out


@dataclass
class KVLayerMixed:
    """Logical cache of one layer whose keys and values have different formats:
    the fp16 tensor as in KVLayerF16 (k or v), the Q8_0 one as in KVLayerQ8
    (kq, ks or vq, vs); the fields of the other format are None."""
    k: Optional[np.ndarray] = None
    kq: Optional[np.ndarray] = None
    ks: Optional[np.ndarray] = None
    v: Optional[np.ndarray] = None
    vq: Optional[np.ndarray] = None
    vs: Optional[np.ndarray] = None


@dataclass
class KVLayerFp8:
    """Logical 8-bit float cache of one layer: kf8, vf8 uint8 E4M3 codes
    [n_slots, n_kv, capacity, head_dim]."""
    kf8: np.ndarray
    vf8: np.ndarray


# Synthetic 8-bit float codes: sign uniform, the other seven bits uniform over
# the 72 codes with exponent field 0..8 (magnitudes up to 3.75, subnormals
# included, never a NaN code).
FP8_CODE_SPAN = 72


def fp8_codes(rng: np.random.Generator, shape) -> np.ndarray:
    low = rng.integers(0, FP8_CODE_SPAN, size=shape, dtype=np.int64)
    sign = rng.integers(0, 2, size=shape, dtype=np.int64)
    return (low | (sign << 7)).astype(np.uint8)


def kv_cache_fp8(rng_k: np.random.Generator, rng_v: np.random.Generator, n_slots: int, n_kv: int,
                 capacity: int, head_dim: int, filled) -> KVLayerFp8:
    shape = (n_slots, n_kv, capacity, head_dim)
    out = KVLayerFp8(kf8=np.zeros(shape, np.uint8), vf8=np.zeros(shape, np.uint8))
    for s in range(n_slots):
        n = int(filled[s])
        out.kf8[s, :, :n] = fp8_codes(rng_k, (n_kv, n, head_dim))
        out.vf8[s, :, :n] = fp8_codes(rng_v, (n_kv, n, head_dim))
    return out


# key / value formats of the cache kinds
KV_FORMATS = {"f16": ("f16", "f16"), "q8_0": ("q8_0", "q8_0"), "q8k_f16v": ("q8_0", "f16"), "f16k_q8v": ("f16", "q8_0"),
              "fp8": ("fp8", "fp8")}


def kv_cache_mixed(rng_k: np.random.Generator, rng_v: np.random.Generator, n_slots: int, n_kv: int,
                   capacity: int, head_dim: int, filled, kind: str) -> KVLayerMixed:
    """Keys and values each drawn as in the cache of their own format (fp16
    N(0,1), or Q8_0 codes uniform in -127..127 with scales |N(0,1)|*0.02),
    keys from rng_k and values from rng_v, slot by slot; zero past filled."""
    shape = (n_slots, n_kv, capacity, head_dim)
    sshape = (n_slots, n_kv, capacity, head_dim // Q8_BLOCK)
    out = KVLayerMixed()
    for name, fmt, rng in (("k", KV_FORMATS[kind][0], rng_k), ("v", KV_FORMATS[kind][1], rng_v)):
        if fmt == "f16":
            t = np.zeros(shape, np.float16)
            for s in range(n_slots):
                n = int(filled[s])
                t[s, :, :n] = f16_normal(rng, (n_kv, n, head_dim))
            setattr(out, name, t)
        else:
            q, sc = np.zeros(shape, np.int8), np.zeros(sshape, np.float16)
            for s in range(n_slots):
                n = int(filled[s])
                q[s, :, :n] = rng.integers(-127, 128, size=(n_kv, n, head_dim), dtype=np.int8)
                sc[s, :, :n] = (np.abs(rng.standard_normal(size=(n_kv, n, head_dim // Q8_BLOCK))) * 0.02).astype(
                    np.float16)
            setattr(out, name + "q", q)
            setattr(out, name + "s", sc)
    return out


def kv_cache(kind: str, rng_k: np.random.Generator, rng_v: np.random.Generator, n_slots: int, n_kv: int,
             capacity: int, head_dim: int, filled):
    """The synthetic cache of a kind: "f16", "q8_0", "q8k_f16v", "f16k_q8v" or "fp8"."""
    if kind == "fp8":
        return kv_cache_fp8(rng_k, rng_v, n_slots, n_kv, capacity, head_dim, filled)
    if kind == "f16":
        return kv_cache_f16(rng_k, rng_v, n_slots, n_kv, capacity, head_dim, filled)
    if kind == "q8_0":
        return kv_cache_q8(rng_k, rng_v, n_slots, n_kv, capacity, head_dim, filled)
    return kv_cache_mixed(rng_k, rng_v, n_slots, n_kv, capacity, head_dim, filled, kind)


def tokens(rng: np.random.Generator, batch: int, vocab: int) -> np.ndarray:
    return rng.integers(0, vocab, size=batch, dtype=np.int64).astype(np.int32)


def ragged_lengths(rng: np.random.Generator, batch: int, lo: int = 512, hi: int = 8192) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=batch).astype(np.int32)
