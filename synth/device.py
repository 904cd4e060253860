"""Seeded synthetic inputs drawn directly on the GPU (torch Philox), for the
multi-gigabyte workloads.  Same distributions as the numpy generators in
synth/__init__.py; like them, this module computes nothing the decode step
computes.  The oracle reads D2H copies of whatever it needs.
"""
from __future__ import annotations

import torch

Q4K_BLOCK_BYTES = 144


def generator(seed: int) -> torch.Generator:
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return g


def q4k_matrix(g: torch.Generator, n_rows: int, n_cols: int) -> torch.Tensor:
    """Random Q4_K matrix bytes (row-tiled order), uint8 tensor of n_rows*n_cols/256*144 bytes."""
    n_blocks = n_rows * (n_cols // 256)
    b = torch.randint(0, 256, (n_blocks, Q4K_BLOCK_BYTES), dtype=torch.uint8, device="cuda", generator=g)
    d = (torch.randn((n_blocks, 2), device="cuda", generator=g).abs() * 1e-3).to(torch.float16)
    b[:, 0:4] = d.view(torch.uint8).view(n_blocks, 4)
    return b.view(-1)


def f16_normal(g: torch.Generator, shape, scale: float = 1.0) -> torch.Tensor:
    x = torch.randn(shape, device="cuda", generator=g)
    if scale != 1.0:
        x = x * scale
    return x.to(torch.float16)


def gains(g: torch.Generator, n: int) -> torch.Tensor:
    return 1.0 + 0.1 * torch.randn(n, device="cuda", generator=g)


def model(dims, seed: int, n_layers=None):
    """(embed, lm_head, norm_final, [layer dicts]) on the GPU for the step ABI."""
    g = generator(seed)
    embed = f16_normal(g, (dims.vocab, dims.hidden))
    lm_head = f16_normal(g, (dims.vocab, dims.hidden), scale=dims.hidden ** -0.5)
    norm_final = gains(g, dims.hidden)
    hq = dims.n_q_heads * dims.head_dim
    layers = []
    for _ in range(dims.n_layers if n_layers is None else n_layers):
        layers.append(dict(w_qkv=q4k_matrix(g, dims.qkv_rows, dims.hidden),
                           w_o=q4k_matrix(g, dims.hidden, hq),
                           w_gate_up=q4k_matrix(g, 2 * dims.ffn, dims.hidden),
                           w_down=q4k_matrix(g, dims.hidden, dims.ffn),
                           norm_attn=gains(g, dims.hidden), norm_ffn=gains(g, dims.hidden)))
    return embed, lm_head, norm_final, layers


def _blocked(vt: torch.Tensor) -> torch.Tensor:
    """Values drawn as [slots, kv, D, cap] -> the cache layout [slots, kv, cap/32, D, 32]."""
    s, k, d, cap = vt.shape
    return vt.reshape(s, k, d, cap // 32, 32).permute(0, 1, 3, 2, 4).contiguous()


def _tensor(g: torch.Generator, fmt: str, shape, filled: int, transposed: bool):
    """One cache tensor (keys [.., cap, D] or transposed values [.., D, cap])
    and its Q8_0 scales ([.., cap, D/32]) or None: fp16 N(0,1), or int8
    uniform in -127..127 with scales |N|*0.02, for positions < filled."""
    n_slots, n_kv, capacity, head_dim = shape
    tshape = (n_slots, n_kv, head_dim, capacity) if transposed else shape
    fill = (n_slots, n_kv, head_dim, filled) if transposed else (n_slots, n_kv, filled, head_dim)
    idx = (slice(None), slice(None), slice(None), slice(0, filled)) if transposed else (
        slice(None), slice(None), slice(0, filled))
    if fmt == "f16":
        t = torch.zeros(tshape, dtype=torch.float16, device="cuda")
        t[idx] = f16_normal(g, fill)
        return t, None
    t = torch.zeros(tshape, dtype=torch.int8, device="cuda")
    t[idx] = torch.randint(-127, 128, fill, dtype=torch.int8, device="cuda", generator=g)
    sc = torch.zeros((n_slots, n_kv, capacity, head_dim // 32), dtype=torch.float16, device="cuda")
    sc[:, :, :filled] = (torch.randn((n_slots, n_kv, filled, head_dim // 32), device="cuda", generator=g).abs()
                         * 0.02).to(torch.float16)
    return t, sc


def kv_cache(g: torch.Generator, kind: str, n_slots: int, n_kv: int, capacity: int, head_dim: int, filled: int):
    """One layer of device cache in the library's layout (values transposed
    within 32-token blocks, drawn as [slots, kv, D, cap] and then blocked),
    N(0,1) fp16 or Q8_0 (int8 uniform in -127..127, scale |N|*0.02) for
    positions < filled and zeros beyond; kind "f16", "q8_0", keys and values
    in different formats, "q8k_f16v" / "f16k_q8v", or "fp8" (uint8 E4M3 codes:
    sign uniform, the other bits uniform over the 72 codes with exponent field
    0..8, as synth.fp8_codes).  Returns (k, v, k_scale, v_scale)."""
    if kind == "fp8":
        def codes(shape):
            low = torch.randint(0, 72, shape, dtype=torch.int32, device="cuda", generator=g)
            sign = torch.randint(0, 2, shape, dtype=torch.int32, device="cuda", generator=g)
            return (low | (sign << 7)).to(torch.uint8)
        k = torch.zeros((n_slots, n_kv, capacity, head_dim), dtype=torch.uint8, device="cuda")
        v = torch.zeros((n_slots, n_kv, head_dim, capacity), dtype=torch.uint8, device="cuda")
        k[:, :, :filled] = codes((n_slots, n_kv, filled, head_dim))
        v[:, :, :, :filled] = codes((n_slots, n_kv, head_dim, filled))
        return k, _blocked(v), None, None
    if kind in ("q8k_f16v", "f16k_q8v"):
        shape = (n_slots, n_kv, capacity, head_dim)
        k, ks = _tensor(g, "q8_0" if kind == "q8k_f16v" else "f16", shape, filled, False)
        v, vs = _tensor(g, "f16" if kind == "q8k_f16v" else "q8_0", shape, filled, True)
        return k, _blocked(v), ks, vs
    if kind == "f16":
        k = torch.zeros((n_slots, n_kv, capacity, head_dim), dtype=torch.float16, device="cuda")
        v = torch.zeros((n_slots, n_kv, head_dim, capacity), dtype=torch.float16, device="cuda")
        k[:, :, :filled] = f16_normal(g, (n_slots, n_kv, filled, head_dim))
        v[:, :, :, :filled] = f16_normal(g, (n_slots, n_kv, head_dim, filled))
        return k, _blocked(v), None, None
    k = torch.zeros((n_slots, n_kv, capacity, head_dim), dtype=torch.int8, device="cuda")
    v = torch.zeros((n_slots, n_kv, head_dim, capacity), dtype=torch.int8, device="cuda")
    ks = torch.zeros((n_slots, n_kv, capacity, head_dim // 32), dtype=torch.float16, device="cuda")
    vs = torch.zeros_like(ks)
    k[:, :, :filled] = torch.randint(-127, 128, (n_slots, n_kv, filled, head_dim), dtype=torch.int8, device="cuda",
                                     generator=g)
    v[:, :, :, :filled] = torch.randint(-127, 128, (n_slots, n_kv, head_dim, filled), dtype=torch.int8, device="cuda",
                                        generator=g)
    ks[:, :, :filled] = (torch.randn((n_slots, n_kv, filled, head_dim // 32), device="cuda", generator=g).abs()
                         * 0.02).to(torch.float16)
    vs[:, :, :filled] = (torch.randn((n_slots, n_kv, filled, head_dim // 32), device="cuda", generator=g).abs()
                         * 0.02).to(torch.float16)
    return k, _blocked(v), ks, vs
