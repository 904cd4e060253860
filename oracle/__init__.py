"""Reference oracle for one batched quantized decode step (TEST INFRASTRUCTURE).

This package is the slow, plain, obviously-correct CPU definition of what the
HIP library computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import it.  It shares no code, constants
or helpers with ``quantized_decode_amd`` and imports nothing from it; the only
thing both sides share is the seeded input generator module ``synth``.

Arithmetic is numpy float64, except at the storage rounding points the method
defines (fp16 activations handed between kernels, fp16 / Q8_0 KV cache
entries), which are rounded exactly as stated in each function.

Sources (three pages of one blog series on batched decode on a single GPU):

* P1: "Batch One Is the Local LLM Assumption Agent Workloads Break on RDNA4"
* P2: "Why a Batched Local Agent Swarm's Speedup Erodes With Context on RDNA4"
* P3: "KV Cache Quantization on RDNA4: Moving the Weight-vs-KV Crossover for a
  Local Agent Swarm"

What pins each part (tests under ``tests/test_oracle_*.py``):

* Q4_K / Q8_0 decoding: hand-built blocks, one-hot bit sweeps, a packer written
  independently of the decoder (bijection), exact rational arithmetic.
* GEMM: exact big-integer matmul in a special case; ``math.fsum`` rows.
* Attention: softmax invariants, n=1, equal keys, GQA == MHA with duplicated
  heads, permutation invariance, log-sum-exp split/merge identity.
* RMSNorm / RoPE / SiLU: closed forms.
* Decode step: batch invariance (bitwise), an identity network that reduces to
  embedding -> final norm -> LM head, and a pure-Python brute force of a
  micro model.  End-to-end logits of the full-size model have no printed
  worked example on the pages: beyond those properties the full-size step is
  "parity unpinned" except through its pinned parts.
* Byte model: the numbers the pages print (tests/golden/pages_numbers.json).
"""
from . import formats, ops, step, bytes_model  # noqa: F401
