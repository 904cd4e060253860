"""Python binding of libqkdec (ctypes).

Every function here only marshals arguments: it takes torch tensors that
already live on the GPU, passes their device pointers and the current HIP
stream to the C ABI of include/qkdec.h, and raises QkdecError on a non-zero
status.  All arithmetic happens in the library's HIP kernels; there is no
fallback path.  Build the library first: ``python -m quantized_decode_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqkdec.so")

GEMM_AUTO = 0           # matvec for B <= MATVEC_AUTO_MAX_B, else the MFMA tiles
GEMM_MFMA = 1
GEMM_MATVEC = 2         # vector-ALU matvec, B <= MATVEC_MAX_B
MATVEC_MAX_B = 2
MATVEC_AUTO_MAX_B = 1

KV_F16 = 0
KV_Q8_0 = 1
KV_Q8_0_K_F16_V = 2     # Q8_0 keys, fp16 values
KV_F16_K_Q8_0_V = 3     # fp16 keys, Q8_0 values
KV_FP8_E4M3 = 4         # OCP E4M3 keys and values, one byte each, no scale
# cache kinds by name (the oracle's names) and their key / value formats
KV_KINDS = {"f16": KV_F16, "q8_0": KV_Q8_0, "q8k_f16v": KV_Q8_0_K_F16_V, "f16k_q8v": KV_F16_K_Q8_0_V,
            "fp8": KV_FP8_E4M3}

STATUS_NAMES = {0: "QKDEC_OK", -1: "QKDEC_E_ARG", -2: "QKDEC_E_SHAPE", -3: "QKDEC_E_ALIGN",
                -4: "QKDEC_E_WORKSPACE", -5: "QKDEC_E_CAPACITY", -6: "QKDEC_E_UNSUPPORTED", -7: "QKDEC_E_HIP"}


class QkdecError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}")
        self.status = status


class KVLayer(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("n_slots", ctypes.c_int32), ("k", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


class Layer(ctypes.Structure):
    _fields_ = [("w_qkv", ctypes.c_void_p), ("w_o", ctypes.c_void_p), ("w_gate_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("norm_attn", ctypes.c_void_p), ("norm_ffn", ctypes.c_void_p)]


class Model(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_base", ctypes.c_float),
                ("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p), ("norm_final", ctypes.c_void_p),
                ("layers", ctypes.POINTER(Layer))]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float

class StepViews(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("x", "h", "qkv", "q16", "o16", "a")]


_SIGNATURES = {
    "qkdec_status_str": (ctypes.c_char_p, [_I32]),
    "qkdec_abi_version": (_I32, []),
    "qkdec_build_id": (ctypes.c_char_p, []),
    "qkdec_gemm_q4k_workspace_size": (_SZ, [_I64, _I64, _I32]),
    "qkdec_gemm_q4k": (_I32, [_P, _I64, _I64, _P, _I64, _I32, _P, _I64, _P, _I64, _P, _SZ, _P]),
    "qkdec_gemm_q4k_xf32": (_I32, [_P, _I64, _I64, _P, _I64, _I32, _P, _I64, _P, _I64, _P, _SZ, _P]),
    "qkdec_gemm_q4k_engine": (_I32, [_P, _I64, _I64, _P, _I64, _I32, _P, _I64, _P, _I64, _I32, _P, _SZ, _P]),
    "qkdec_gemm_q4k_swiglu_workspace_size": (_SZ, [_I64, _I64, _I32]),
    "qkdec_gemm_q4k_swiglu": (_I32, [_P, _I64, _I64, _P, _I64, _I32, _P, _I64, _P, _SZ, _P]),
    "qkdec_dequant_q4k": (_I32, [_P, _I64, _P, _P]),
    "qkdec_kv_append_f16": (_I32, [ctypes.POINTER(KVLayer), _P, _P, _P, _P, _I32, _P, _P]),
    "qkdec_kv_append_q8_0": (_I32, [ctypes.POINTER(KVLayer), _P, _P, _P, _P, _I32, _P, _P]),
    "qkdec_kv_append": (_I32, [ctypes.POINTER(KVLayer), _P, _P, _P, _P, _I32, _P, _P]),
    "qkdec_attn_workspace_size": (_SZ, [_I32, _I32, ctypes.POINTER(KVLayer)]),
    "qkdec_attn_decode": (_I32, [ctypes.POINTER(KVLayer), _P, _P, _I32, _P, _I32, _F, _P, _P, _P, _SZ, _P]),
    "qkdec_attn_paged_workspace_size": (_SZ, [_I32, _I32, ctypes.POINTER(KVLayer), _I32]),
    "qkdec_attn_decode_paged": (_I32, [ctypes.POINTER(KVLayer), _P, _I32, _P, _I32, _P, _I32, _F, _P, _P, _P, _SZ,
                                       _P]),
    "qkdec_kv_append_paged": (_I32, [ctypes.POINTER(KVLayer), _P, _I32, _P, _P, _P, _I32, _P, _P]),
    "qkdec_lm_head_workspace_size": (_SZ, [_I64, _I32]),
    "qkdec_lm_head_argmax": (_I32, [_P, _I64, _I64, _P, _I32, _P, _P, _P, _SZ, _P]),
    "qkdec_step_workspace_size": (_SZ, [ctypes.POINTER(Model), _I32, ctypes.POINTER(KVLayer)]),
    "qkdec_workspace_init": (_I32, [_P, _SZ, _P]),
    "qkdec_step": (_I32, [ctypes.POINTER(Model), ctypes.POINTER(KVLayer), _P, _P, _P, _I32, _P, _P, _SZ, _P]),
    "qkdec_step_status": (_I32, [_P, _P]),
    "qkdec_prefill_workspace_size": (_SZ, [ctypes.POINTER(Model), ctypes.POINTER(KVLayer)]),
    "qkdec_prefill": (_I32, [ctypes.POINTER(Model), ctypes.POINTER(KVLayer), _I32, _I32, _P, _I32, _P, _P, _P, _SZ,
                             _P]),
    "qkdec_prefill_paged_workspace_size": (_SZ, [ctypes.POINTER(Model), ctypes.POINTER(KVLayer)]),
    "qkdec_prefill_paged": (_I32, [ctypes.POINTER(Model), ctypes.POINTER(KVLayer), _P, _I32, _I32, _P, _I32, _P, _P,
                                   _P, _SZ, _P]),
    "qkdec_step_noalloc_max_bytes": (_SZ, []),
    "qkdec_step_noalloc": (_I32, [ctypes.POINTER(Model), ctypes.POINTER(KVLayer), _P, _P, _P, _I32, _P, _P, _P]),
    "qkdec_step_paged_workspace_size": (_SZ, [ctypes.POINTER(Model), _I32, ctypes.POINTER(KVLayer), _I32]),
    "qkdec_step_paged": (_I32, [ctypes.POINTER(Model), ctypes.POINTER(KVLayer), _P, _I32, _P, _P, _I32, _P, _P, _SZ,
                                _P]),
    "qkdec_step_workspace_views": (_I32, [ctypes.POINTER(Model), _I32, ctypes.POINTER(KVLayer),
                                          ctypes.POINTER(StepViews)]),
    "qkdec_plan_create": (_I32, [ctypes.POINTER(_P), ctypes.POINTER(Model), ctypes.POINTER(KVLayer), _P, _P, _P,
                                 _I32, _P, _P, _SZ, _P]),
    "qkdec_plan_launch": (_I32, [_P, _P]),
    "qkdec_plan_destroy": (None, [_P]),
}

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libqkdec.so (once) and declare every entry point's signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m quantized_decode_amd.build`")
    # torch ships its own libamdhip64.so.7.  Loading it first makes the library's
    # dependency of the same soname resolve to that copy; loaded the other way
    # round, the process holds two HIP runtimes and launches on torch's memory fail.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise QkdecError(status, where)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# ------------------------------------------------------------------ entry points
def qkdec_build_id() -> str:
    """The build id of the loaded library (hash of the sources it was built from)."""
    return load_library().qkdec_build_id().decode()


def qkdec_gemm_q4k_workspace_size(n: int, k: int, b: int) -> int:
    return load_library().qkdec_gemm_q4k_workspace_size(n, k, b)


def qkdec_gemm_q4k(w, n: int, k: int, x, b: int, y, residual=None, workspace=None, stream=None) -> None:
    """y[:b, :n] = residual + x[:b, :k] @ deq(w).T  (x fp16 [b, ldx], y fp32 [b, ldy])."""
    lib = load_library()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.qkdec_gemm_q4k(_ptr(w), n, k, _ptr(x), x.stride(0), b, _ptr(y), y.stride(0), _ptr(residual),
                              residual.stride(0) if residual is not None else 0, _ptr(workspace), ws_bytes,
                              _stream(stream)), "qkdec_gemm_q4k")


def qkdec_gemm_q4k_engine(w, n: int, k: int, x, b: int, y, engine: int, residual=None, workspace=None,
                          stream=None) -> None:
    """qkdec_gemm_q4k with the engine chosen (GEMM_AUTO, GEMM_MFMA or GEMM_MATVEC)."""
    lib = load_library()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.qkdec_gemm_q4k_engine(_ptr(w), n, k, _ptr(x), x.stride(0), b, _ptr(y), y.stride(0), _ptr(residual),
                                     residual.stride(0) if residual is not None else 0, engine, _ptr(workspace),
                                     ws_bytes, _stream(stream)), "qkdec_gemm_q4k_engine")


def qkdec_gemm_q4k_xf32(w, n: int, k: int, x, b: int, y, residual=None, workspace=None, stream=None) -> None:
    """As qkdec_gemm_q4k with fp32 x, rounded in-kernel to fp16 per 256-value block."""
    lib = load_library()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.qkdec_gemm_q4k_xf32(_ptr(w), n, k, _ptr(x), x.stride(0), b, _ptr(y), y.stride(0), _ptr(residual),
                                   residual.stride(0) if residual is not None else 0, _ptr(workspace), ws_bytes,
                                   _stream(stream)), "qkdec_gemm_q4k_xf32")


def qkdec_gemm_q4k_swiglu_workspace_size(f: int, k: int, b: int) -> int:
    return load_library().qkdec_gemm_q4k_swiglu_workspace_size(f, k, b)


def qkdec_gemm_q4k_swiglu(w, f: int, k: int, x, b: int, a, workspace=None, stream=None) -> None:
    """a[:b, :f] = silu(x W_gate^T) * (x W_up^T) (fp32) with w holding 2f rows."""
    lib = load_library()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.qkdec_gemm_q4k_swiglu(_ptr(w), f, k, _ptr(x), x.stride(0), b, _ptr(a), a.stride(0),
                                     _ptr(workspace), ws_bytes, _stream(stream)), "qkdec_gemm_q4k_swiglu")


def qkdec_dequant_q4k(w, n_blocks: int, out, stream=None) -> None:
    _check(load_library().qkdec_dequant_q4k(_ptr(w), n_blocks, _ptr(out), _stream(stream)), "qkdec_dequant_q4k")


def kv_layer(kind: int, n_kv_heads: int, head_dim: int, capacity: int, n_slots: int, k, v,
             k_scale=None, v_scale=None) -> KVLayer:
    return KVLayer(kind, n_kv_heads, head_dim, capacity, n_slots, _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale))


def qkdec_kv_append_f16(kv: KVLayer, slot, pos, k, v, b: int, err=None, stream=None) -> None:
    _check(load_library().qkdec_kv_append_f16(ctypes.byref(kv), _ptr(slot), _ptr(pos), _ptr(k), _ptr(v), b,
                                              _ptr(err), _stream(stream)), "qkdec_kv_append_f16")


def qkdec_kv_append_q8_0(kv: KVLayer, slot, pos, k, v, b: int, err=None, stream=None) -> None:
    _check(load_library().qkdec_kv_append_q8_0(ctypes.byref(kv), _ptr(slot), _ptr(pos), _ptr(k), _ptr(v), b,
                                               _ptr(err), _stream(stream)), "qkdec_kv_append_q8_0")


def qkdec_kv_append(kv: KVLayer, slot, pos, k, v, b: int, err=None, stream=None) -> None:
    _check(load_library().qkdec_kv_append(ctypes.byref(kv), _ptr(slot), _ptr(pos), _ptr(k), _ptr(v), b,
                                          _ptr(err), _stream(stream)), "qkdec_kv_append")


def qkdec_attn_workspace_size(b: int, n_q_heads: int, kv: KVLayer) -> int:
    return load_library().qkdec_attn_workspace_size(b, n_q_heads, ctypes.byref(kv))


def qkdec_attn_decode(kv: KVLayer, slot, n_ctx, b: int, q, n_q_heads: int, scale: float, o=None, o16=None,
                      workspace=None, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().qkdec_attn_decode(ctypes.byref(kv), _ptr(slot), _ptr(n_ctx), b, _ptr(q), n_q_heads,
                                            scale, _ptr(o), _ptr(o16), _ptr(workspace), ws_bytes,
                                            _stream(stream)), "qkdec_attn_decode")


def qkdec_attn_paged_workspace_size(b: int, n_q_heads: int, kv: KVLayer, max_pages: int) -> int:
    return load_library().qkdec_attn_paged_workspace_size(b, n_q_heads, ctypes.byref(kv), max_pages)


def qkdec_attn_decode_paged(kv: KVLayer, pages, max_pages: int, n_ctx, b: int, q, n_q_heads: int, scale: float,
                            o=None, o16=None, workspace=None, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().qkdec_attn_decode_paged(ctypes.byref(kv), _ptr(pages), max_pages, _ptr(n_ctx), b, _ptr(q),
                                                  n_q_heads, scale, _ptr(o), _ptr(o16), _ptr(workspace), ws_bytes,
                                                  _stream(stream)), "qkdec_attn_decode_paged")


def qkdec_kv_append_paged(kv: KVLayer, pages, max_pages: int, pos, k, v, b: int, err=None, stream=None) -> None:
    _check(load_library().qkdec_kv_append_paged(ctypes.byref(kv), _ptr(pages), max_pages, _ptr(pos), _ptr(k), _ptr(v),
                                                b, _ptr(err), _stream(stream)), "qkdec_kv_append_paged")


def qkdec_lm_head_workspace_size(vocab: int, b: int) -> int:
    return load_library().qkdec_lm_head_workspace_size(vocab, b)


def qkdec_lm_head_argmax(w, vocab: int, hidden: int, x, b: int, tok, logits=None, workspace=None,
                         stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().qkdec_lm_head_argmax(_ptr(w), vocab, hidden, _ptr(x), b, _ptr(logits), _ptr(tok),
                                               _ptr(workspace), ws_bytes, _stream(stream)), "qkdec_lm_head_argmax")


class StepModel:
    """Holds the ctypes model descriptor (and keeps its host arrays alive)."""

    def __init__(self, dims, embed, lm_head, norm_final, layers: Sequence[dict], kv_layers: List[KVLayer]):
        self.layer_arr = (Layer * len(layers))(*[
            Layer(_ptr(l["w_qkv"]), _ptr(l["w_o"]), _ptr(l["w_gate_up"]), _ptr(l["w_down"]),
                  _ptr(l["norm_attn"]), _ptr(l["norm_ffn"])) for l in layers])
        self.model = Model(len(layers), dims.hidden, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.ffn,
                           dims.vocab, dims.rms_eps, dims.rope_base, _ptr(embed), _ptr(lm_head), _ptr(norm_final),
                           ctypes.cast(self.layer_arr, ctypes.POINTER(Layer)))
        self.kv_layers = list(kv_layers)
        self.kv_arr = (KVLayer * len(kv_layers))(*kv_layers)


def qkdec_step_workspace_size(sm: StepModel, b: int) -> int:
    return load_library().qkdec_step_workspace_size(ctypes.byref(sm.model), b, sm.kv_arr)


def qkdec_workspace_init(workspace, stream=None) -> None:
    _check(load_library().qkdec_workspace_init(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                               _stream(stream)), "qkdec_workspace_init")


def qkdec_step(sm: StepModel, slot, pos, tok, b: int, workspace, logits=None, stream=None) -> None:
    _check(load_library().qkdec_step(ctypes.byref(sm.model), sm.kv_arr, _ptr(slot), _ptr(pos), _ptr(tok), b,
                                     _ptr(logits), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream)), "qkdec_step")


def qkdec_step_paged_workspace_size(sm: StepModel, b: int, max_pages: int) -> int:
    return load_library().qkdec_step_paged_workspace_size(ctypes.byref(sm.model), b, sm.kv_arr, max_pages)


def qkdec_step_paged(sm: StepModel, pages, max_pages: int, pos, tok, b: int, workspace, logits=None,
                     stream=None) -> None:
    _check(load_library().qkdec_step_paged(ctypes.byref(sm.model), sm.kv_arr, _ptr(pages), max_pages, _ptr(pos),
                                           _ptr(tok), b, _ptr(logits), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream(stream)),
           "qkdec_step_paged")


def qkdec_prefill_workspace_size(sm: StepModel) -> int:
    return load_library().qkdec_prefill_workspace_size(ctypes.byref(sm.model), sm.kv_arr)


def qkdec_prefill(sm: StepModel, slot: int, start: int, tokens, n: int, tok_out, workspace, logits=None,
                  stream=None) -> None:
    """Append prompt tokens (device int32 [n]) at positions start.. of slot;
    tok_out (device int32 [1]) gets the argmax after the last one."""
    _check(load_library().qkdec_prefill(ctypes.byref(sm.model), sm.kv_arr, slot, start, _ptr(tokens), n,
                                        _ptr(logits), _ptr(tok_out), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream)),
           "qkdec_prefill")


def qkdec_prefill_paged_workspace_size(sm: StepModel) -> int:
    return load_library().qkdec_prefill_paged_workspace_size(ctypes.byref(sm.model), sm.kv_arr)


def qkdec_prefill_paged(sm: StepModel, pages, max_pages: int, start: int, tokens, n: int, tok_out, workspace,
                        logits=None, stream=None) -> None:
    """Append prompt tokens (device int32 [n]) at positions start.. of the
    sequence whose page table row is pages (device int32 [max_pages]) in
    every layer's paged pool; tok_out gets the argmax after the last one."""
    _check(load_library().qkdec_prefill_paged(ctypes.byref(sm.model), sm.kv_arr, _ptr(pages), max_pages, start,
                                              _ptr(tokens), n, _ptr(logits), _ptr(tok_out), _ptr(workspace),
                                              workspace.numel() * workspace.element_size(), _stream(stream)),
           "qkdec_prefill_paged")


def qkdec_step_noalloc_max_bytes() -> int:
    return load_library().qkdec_step_noalloc_max_bytes()


def qkdec_step_noalloc(sm: StepModel, slot, pos, tok, b: int, err, logits=None, stream=None) -> None:
    """qkdec_step without a workspace (the library's fixed device scratch);
    err: device int32 [1], set to QKDEC_E_CAPACITY on a full cache."""
    _check(load_library().qkdec_step_noalloc(ctypes.byref(sm.model), sm.kv_arr, _ptr(slot), _ptr(pos), _ptr(tok), b,
                                             _ptr(logits), _ptr(err), _stream(stream)), "qkdec_step_noalloc")


def qkdec_step_status(workspace, stream=None) -> int:
    return load_library().qkdec_step_status(_ptr(workspace), _stream(stream))


def qkdec_step_workspace_views(sm: StepModel, b: int) -> dict:
    """Byte offsets of the last layer's stage outputs inside a step workspace."""
    v = StepViews()
    _check(load_library().qkdec_step_workspace_views(ctypes.byref(sm.model), b, sm.kv_arr, ctypes.byref(v)),
           "qkdec_step_workspace_views")
    return {n: getattr(v, n) for n, _ in StepViews._fields_}


class Plan:
    """A captured decode step (qkdec_plan_create / _launch / _destroy)."""

    def __init__(self, sm: StepModel, slot, pos, tok, b: int, workspace, logits=None, stream=None):
        self._sm = sm
        self._keep = (slot, pos, tok, workspace, logits)
        self.handle = ctypes.c_void_p()
        _check(load_library().qkdec_plan_create(ctypes.byref(self.handle), ctypes.byref(sm.model), sm.kv_arr,
                                                _ptr(slot), _ptr(pos), _ptr(tok), b, _ptr(logits), _ptr(workspace),
                                                workspace.numel() * workspace.element_size(), _stream(stream)),
               "qkdec_plan_create")

    def launch(self, stream=None) -> None:
        _check(load_library().qkdec_plan_launch(self.handle, _stream(stream)), "qkdec_plan_launch")

    def destroy(self) -> None:
        if self.handle:
            load_library().qkdec_plan_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass
