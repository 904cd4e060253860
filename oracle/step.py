"""One batched decode step in plain fp64 (oracle; test infrastructure only).
(P1, P2, P3: the three pages listed, with their titles, in oracle/__init__.py.)

P1 "The weight read is the only term that does not scale" and P2 "The two
halves of a decode-step memory bill" describe the step: the weights are
streamed once and multiplied against every sequence's hidden state; each
sequence reads its own whole KV cache; norms and SwiGLU process one row per
sequence; the LM head matmul and the (greedy) sampling are per sequence.

Model: a pre-norm decoder.  Per layer
    h  = f16(RMSNorm(x))             ; [q;k;v] = h W_qkv^T
    q, k = RoPE(q, k, pos)           ; append f16(k), f16(v) (or Q8_0) at pos
    O  = Attention(f16(q), cache[0..pos])  ; x += f16(O) W_o^T
    h2 = f16(RMSNorm(x))             ; x += f16b(silu(h2 W_g^T) * (h2 W_u^T)) W_d^T
then hf = f16(RMSNorm_final(x)), logits = hf W_lm^T, token = argmax (lowest
index on ties).  f16(.) is round-to-nearest-even to fp16; f16b(.) is the same
with one power-of-two exponent offset per 256 values (formats.round_f16_blocked)
so that the SwiGLU activation cannot overflow; everything else is fp64.
The model object needs attributes dims, embed, lm_head, norm_final and
layers[i].{w_qkv, w_o, w_gate_up, w_down, norm_attn, norm_ffn}; caches are per
layer with k, (kq, ks) or kf8 for the keys and v, (vq, vs) or vf8 for the
values (fp16, Q8_0 codes and scales, or E4M3 codes), arrays of logical shape [n_slots, n_kv, capacity,
head_dim] (scales [.., head_dim/32]).
"""
from __future__ import annotations

import numpy as np

from .formats import (fp8_e4m3_decode, fp8_e4m3_encode, q8_0_dequant, q8_0_quantize, round_f16,
                      round_f16_blocked)
from .ops import argmax_lowest, attention, dense_gemm, q4k_gemm, rmsnorm, rope, swiglu


# Key and value formats of each cache kind.  P3 "Why Q8 is close to free and
# where the sharp edges are" and its FAQ "Does KV cache quantization hurt
# output quality?": keys and values take their formats independently.  "fp8":
# both in the 8-bit float format of formats.fp8_e4m3_encode (P2 "What a
# long-running swarm should actually tune").
KV_FORMATS = {"f16": ("f16", "f16"), "q8_0": ("q8_0", "q8_0"),
              "q8k_f16v": ("q8_0", "f16"), "f16k_q8v": ("f16", "q8_0"), "fp8": ("fp8", "fp8")}


def kv_append(cache, kind: str, slot: int, pos: int, k: np.ndarray, v: np.ndarray) -> None:
    """Store one token's keys and values ([n_kv, D], fp64) at index pos of slot.

    Each tensor in its own format (KV_FORMATS[kind]).  fp16: round to
    nearest-even fp16 (fields k / v).  Q8_0 (P3 "Why Q8 is close to free and
    where the sharp edges are"): per 32 values of one token and head, see
    formats.q8_0_quantize (fields kq, ks / vq, vs).  fp8: one E4M3 code per
    value, formats.fp8_e4m3_encode (fields kf8 / vf8).
    """
    if kind not in KV_FORMATS:
        raise ValueError(kind)
    for name, fmt, x in (("k", KV_FORMATS[kind][0], k), ("v", KV_FORMATS[kind][1], v)):
        if fmt == "f16":
            getattr(cache, name)[slot, :, pos] = np.asarray(x, dtype=np.float64).astype(np.float16)
        elif fmt == "fp8":
            getattr(cache, name + "f8")[slot, :, pos] = fp8_e4m3_encode(x)
        else:
            q, d = q8_0_quantize(x)
            getattr(cache, name + "q")[slot, :, pos] = q
            getattr(cache, name + "s")[slot, :, pos] = d


def kv_read(cache, kind: str, slot: int, n: int):
    """Keys and values of the first n positions of slot as fp64 [n_kv, n, D].

    P3 (FAQ "Is KV cache quantization a kernel change or a storage change?"):
    the attention reads the quantized values dequantized, d*q.
    """
    if kind not in KV_FORMATS:
        raise ValueError(kind)
    out = []
    for name, fmt in (("k", KV_FORMATS[kind][0]), ("v", KV_FORMATS[kind][1])):
        if fmt == "f16":
            out.append(getattr(cache, name)[slot, :, :n].astype(np.float64))
        elif fmt == "fp8":
            out.append(fp8_e4m3_decode(getattr(cache, name + "f8")[slot, :, :n]))
        else:
            out.append(q8_0_dequant(getattr(cache, name + "q")[slot, :, :n], getattr(cache, name + "s")[slot, :, :n]))
    return out[0], out[1]


def _attend(q: np.ndarray, kd: np.ndarray, vd: np.ndarray, scale: float) -> np.ndarray:
    """attention() of one sequence; a sequence with no cached token gets O = 0."""
    if kd.shape[1] == 0:
        return np.zeros(q.shape, dtype=np.float64)
    return attention(q, kd, vd, scale)


def attention_batch(q: np.ndarray, cache, kind: str, slots, n_ctx, scale: float) -> np.ndarray:
    """Standalone decode attention: q [B, Hq, D] against n_ctx[b] cached tokens
    of slot[b] (n_ctx[b] <= 0: O = 0)."""
    out = np.empty(q.shape, dtype=np.float64)
    for b in range(q.shape[0]):
        kd, vd = kv_read(cache, kind, int(slots[b]), max(0, int(n_ctx[b])))
        out[b] = _attend(q[b], kd, vd, scale)
    return out


# ---- paged cache (P1 "Where it stops, and the argument I got wrong in May":
# sequences of very different lengths share one pool of fixed-size pages,
# admitted and released between decode steps).  A pool is a cache object of
# the layout above whose "slots" are pages of page_tokens positions each;
# sequence b's token t lives in page pages[b][t // page_tokens] at offset
# t % page_tokens.  A table entry outside the pool (-1: no page handed out)
# maps nothing: the tokens it would hold are not part of the sequence's
# context (reading skips them, a store to them is dropped).


def _pool_pages(pool) -> int:
    for name in ("k", "kq", "kf8"):
        arr = getattr(pool, name, None)
        if arr is not None:
            return arr.shape[0]
    raise ValueError("pool without keys")


def kv_read_paged(pool, kind: str, pages, page_tokens: int, n: int):
    """Keys and values of the mapped tokens among the first n of a paged
    sequence, in order, fp64 [n_kv, n_mapped, D]."""
    n_pages = _pool_pages(pool)
    ks, vs = [kv_read(pool, kind, 0, 0)[0]], [kv_read(pool, kind, 0, 0)[1]]
    for i in range((max(0, n) + page_tokens - 1) // page_tokens):
        pg = int(pages[i])
        if not 0 <= pg < n_pages:
            continue
        take = min(page_tokens, n - i * page_tokens)
        kd, vd = kv_read(pool, kind, pg, take)
        ks.append(kd)
        vs.append(vd)
    return np.concatenate(ks, axis=1), np.concatenate(vs, axis=1)


def kv_append_paged(pool, kind: str, pages, page_tokens: int, pos: int, k: np.ndarray, v: np.ndarray) -> bool:
    """kv_append of one token at logical position pos of a paged sequence;
    False (nothing stored) when pos lies outside the table or on an unmapped page."""
    i = pos // page_tokens
    if pos < 0 or i >= len(pages) or not 0 <= int(pages[i]) < _pool_pages(pool):
        return False
    kv_append(pool, kind, int(pages[i]), pos % page_tokens, k, v)
    return True


def attention_batch_paged(q: np.ndarray, pool, kind: str, page_table, page_tokens: int, n_ctx,
                          scale: float) -> np.ndarray:
    """attention_batch over paged sequences: page_table[b] lists sequence b's
    pages in order; tokens on unmapped pages are left out of the softmax and a
    sequence with no mapped token gets O = 0."""
    out = np.empty(q.shape, dtype=np.float64)
    for b in range(q.shape[0]):
        kd, vd = kv_read_paged(pool, kind, page_table[b], page_tokens, int(n_ctx[b]))
        out[b] = _attend(q[b], kd, vd, scale)
    return out


def decode_step(model, caches, kind: str, slots, pos, tok, n_layers=None):
    """Advance every sequence by one token.

    Appends this step's keys/values to ``caches`` (mutated) at pos[b] and
    attends over pos[b]+1 tokens.  Returns (logits fp64 [B, vocab], next token
    int64 [B]); the caller advances pos by one.
    """
    def append(cache, b, p, k, v):
        kv_append(cache, kind, int(slots[b]), p, k, v)

    def read(cache, b, n):
        return kv_read(cache, kind, int(slots[b]), n)

    return _step(model, caches, pos, tok, append, read, n_layers)


def decode_step_paged(model, pools, kind: str, page_table, page_tokens: int, pos, tok, n_layers=None):
    """decode_step over paged pools (one per layer, all sharing page_table:
    sequence b's token t sits in page page_table[b][t // page_tokens] of every
    layer).  The new token goes to position pos[b] of sequence b (dropped when
    its page is unmapped, kv_append_paged); attention reads the mapped tokens
    among the first pos[b]+1."""
    def append(pool, b, p, k, v):
        kv_append_paged(pool, kind, page_table[b], page_tokens, p, k, v)

    def read(pool, b, n):
        return kv_read_paged(pool, kind, page_table[b], page_tokens, n)

    return _step(model, pools, pos, tok, append, read, n_layers)


def _step(model, caches, pos, tok, append, read, n_layers):
    dm = model.dims
    hq, hkv, hd = dm.n_q_heads, dm.n_kv_heads, dm.head_dim
    f = dm.ffn
    qrows, krows = hq * hd, hkv * hd
    tok = np.asarray(tok, dtype=np.int64)
    bsz = tok.shape[0]
    scale = 1.0 / np.sqrt(hd)
    x = model.embed[tok].astype(np.float64)
    layers = model.layers if n_layers is None else model.layers[:n_layers]
    for li, ly in enumerate(layers):
        cache = caches[li]
        h = round_f16(rmsnorm(x, ly.norm_attn, dm.rms_eps))
        qkv = q4k_gemm(ly.w_qkv, qrows + 2 * krows, dm.hidden, h)
        o = np.empty((bsz, qrows), dtype=np.float64)
        for b in range(bsz):
            p = int(pos[b])
            q = rope(qkv[b, :qrows].reshape(hq, hd), p, dm.rope_base)
            k = rope(qkv[b, qrows:qrows + krows].reshape(hkv, hd), p, dm.rope_base)
            v = qkv[b, qrows + krows:].reshape(hkv, hd)
            append(cache, b, p, k, v)
            kd, vd = read(cache, b, p + 1)
            o[b] = _attend(round_f16(q), kd, vd, scale).reshape(-1)
        x = x + q4k_gemm(ly.w_o, dm.hidden, qrows, round_f16(o))
        h2 = round_f16(rmsnorm(x, ly.norm_ffn, dm.rms_eps))
        gu = q4k_gemm(ly.w_gate_up, 2 * f, dm.hidden, h2)
        a = round_f16_blocked(swiglu(gu[:, :f], gu[:, f:]))
        x = x + q4k_gemm(ly.w_down, dm.hidden, f, a)
    hf = round_f16(rmsnorm(x, model.norm_final, dm.rms_eps))
    logits = dense_gemm(model.lm_head, hf)
    return logits, argmax_lowest(logits)


def prefill(model, caches, kind: str, slot: int, start: int, tokens):
    """Ingest a prompt into one sequence's cache (P2 "This is the mirror image
    of the prefill story").  By definition this is the decode step applied to
    the prompt's tokens in order: token i sits at position start + i, its keys
    and values are appended, and it attends over every earlier position and
    itself.  Mutates ``caches``; returns (logits fp64 [vocab] after the last
    token, their argmax)."""
    logits, nt = None, None
    for i, t in enumerate(tokens):
        logits, nt = decode_step(model, caches, kind, [slot], [start + i], [int(t)])
    return logits[0], int(nt[0])
