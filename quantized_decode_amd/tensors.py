"""Device-memory helpers: lay host arrays out in the library's storage formats.

These only move and reorder bytes (torch is used for device memory); the one
layout change is the value cache, which the library keeps transposed within
blocks of 32 tokens per head ([slot][kv head][capacity/32][head_dim][32]).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import KV_F16, KV_F16_K_Q8_0_V, KV_FP8_E4M3, KV_Q8_0, KV_Q8_0_K_F16_V, KVLayer, kv_layer


def dev(a: np.ndarray):
    """numpy -> contiguous CUDA tensor with the same bytes and dtype."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to("cuda")


def empty(shape, dtype):
    import torch
    return torch.empty(shape, dtype=dtype, device="cuda")


def v_to_blocked(v: np.ndarray) -> np.ndarray:
    """Logical values [slots, kv, cap, D] -> the cache layout [slots, kv, cap/32, D, 32]."""
    s, k, cap, d = v.shape
    return np.ascontiguousarray(v.reshape(s, k, cap // 32, 32, d).transpose(0, 1, 2, 4, 3))


def v_from_blocked(vb: np.ndarray) -> np.ndarray:
    """The cache layout [slots, kv, cap/32, D, 32] -> logical values [slots, kv, cap, D]."""
    s, k, t, d, _ = vb.shape
    return np.ascontiguousarray(vb.transpose(0, 1, 2, 4, 3).reshape(s, k, t * 32, d))


@dataclass
class DeviceKV:
    """One layer of device KV cache plus its ctypes descriptor."""
    kind: int
    k: object
    v: object                 # transposed in 32-token blocks: [slots][kv][cap/32][D][32]
    k_scale: Optional[object]
    v_scale: Optional[object]
    desc: KVLayer

    def logical_f16(self):
        """(k, v) as numpy fp16 [slots, kv, cap, D] (v transposed back)."""
        return self.k.cpu().numpy(), v_from_blocked(self.v.cpu().numpy())

    def logical_q8(self):
        kq = self.k.cpu().numpy()
        vq = v_from_blocked(self.v.cpu().numpy())
        return kq, self.k_scale.cpu().numpy(), vq, self.v_scale.cpu().numpy()

    def set_v_from(self, slot: int, first: int, value) -> None:
        """Set every value of positions >= first of slot (all heads and dims)."""
        t0, j0 = divmod(first, 32)
        if j0:
            self.v[slot, :, t0, :, j0:] = value
            t0 += 1
        self.v[slot, :, t0:] = value

    def logical(self):
        """The cache as a logical object with the fields of its formats: k,
        (kq, ks) or kf8, v, (vq, vs) or vf8, numpy [slots, kv, cap, D] (v
        transposed back)."""
        from types import SimpleNamespace
        k = self.k.cpu().numpy()
        v = v_from_blocked(self.v.cpu().numpy())
        out = SimpleNamespace()
        if self.kind == KV_FP8_E4M3:
            out.kf8, out.vf8 = k, v
            return out
        if self.k_scale is None:
            out.k = k
        else:
            out.kq, out.ks = k, self.k_scale.cpu().numpy()
        if self.v_scale is None:
            out.v = v
        else:
            out.vq, out.vs = v, self.v_scale.cpu().numpy()
        return out


def _f16_t(a):
    import torch
    return dev(np.ascontiguousarray(a).view(np.uint16)).view(torch.float16)


def upload_kv_f16(k: np.ndarray, v: np.ndarray) -> DeviceKV:
    """k, v: fp16 [slots, kv, cap, D] (logical)."""
    slots, nkv, cap, d = k.shape
    kd = _f16_t(k)
    vd = _f16_t(v_to_blocked(v))
    return DeviceKV(KV_F16, kd, vd, None, None, kv_layer(KV_F16, nkv, d, cap, slots, kd, vd))


def upload_kv_q8(kq: np.ndarray, ks: np.ndarray, vq: np.ndarray, vs: np.ndarray) -> DeviceKV:
    """kq, vq: int8 [slots, kv, cap, D]; ks, vs: fp16 [slots, kv, cap, D/32] (logical)."""
    slots, nkv, cap, d = kq.shape
    kd = dev(kq)
    vd = dev(v_to_blocked(vq))
    ksd, vsd = _f16_t(ks), _f16_t(vs)
    return DeviceKV(KV_Q8_0, kd, vd, ksd, vsd, kv_layer(KV_Q8_0, nkv, d, cap, slots, kd, vd, ksd, vsd))


def upload_kv_fp8(kf8: np.ndarray, vf8: np.ndarray) -> DeviceKV:
    """kf8, vf8: uint8 E4M3 codes [slots, kv, cap, D] (logical)."""
    slots, nkv, cap, d = kf8.shape
    kd = dev(np.asarray(kf8, dtype=np.uint8))
    vd = dev(v_to_blocked(np.asarray(vf8, dtype=np.uint8)))
    return DeviceKV(KV_FP8_E4M3, kd, vd, None, None, kv_layer(KV_FP8_E4M3, nkv, d, cap, slots, kd, vd))


def upload_cache(c) -> DeviceKV:
    """A logical cache object with k, (kq, ks) or kf8 for the keys and v,
    (vq, vs) or vf8 for the values; fields of the other formats absent or None."""
    if getattr(c, "kf8", None) is not None:
        return upload_kv_fp8(c.kf8, c.vf8)
    kq8 = getattr(c, "kq", None) is not None
    vq8 = getattr(c, "vq", None) is not None
    if kq8 and vq8:
        return upload_kv_q8(c.kq, c.ks, c.vq, c.vs)
    if not kq8 and not vq8:
        return upload_kv_f16(c.k, c.v)
    kl = c.kq if kq8 else c.k
    slots, nkv, cap, d = kl.shape
    kd = dev(c.kq) if kq8 else _f16_t(c.k)
    ksd = _f16_t(c.ks) if kq8 else None
    vd = dev(v_to_blocked(c.vq)) if vq8 else _f16_t(v_to_blocked(c.v))
    vsd = _f16_t(c.vs) if vq8 else None
    kind = KV_Q8_0_K_F16_V if kq8 else KV_F16_K_Q8_0_V
    return DeviceKV(kind, kd, vd, ksd, vsd, kv_layer(kind, nkv, d, cap, slots, kd, vd, ksd, vsd))


def upload_model(model):
    """Device tensors of a synthetic model: (embed, lm_head, norm_final, [layer dicts])."""
    import torch
    layers = [dict(w_qkv=dev(l.w_qkv.reshape(-1)), w_o=dev(l.w_o.reshape(-1)),
                   w_gate_up=dev(l.w_gate_up.reshape(-1)), w_down=dev(l.w_down.reshape(-1)),
                   norm_attn=dev(l.norm_attn), norm_ffn=dev(l.norm_ffn)) for l in model.layers]
    return (_f16_t(model.embed), _f16_t(model.lm_head), dev(model.norm_final), layers)
