"""Python binding of the qdec C ABI (include/qdec.h): argument marshalling only.

Every function has the C name and raises QdecError(code, message) when the C
call returns a non-zero status. Device buffers are passed as integer device
addresses (e.g. ``tensor.data_ptr()`` of a torch tensor on the GPU); streams
as ``torch.cuda.current_stream().cuda_stream``. The library must have been
built (``python -m qwen3_kv_cache_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqdec.so")

QDEC_OK = 0
QDEC_E_INVALID = -1
QDEC_E_POS = -2
QDEC_E_CAPACITY = -3
QDEC_E_STATE = -4
QDEC_E_OOM = -5
QDEC_E_DEVICE = -6

QDEC_F32 = 0
QDEC_BF16 = 1
QDEC_Q8_0 = 2
QDEC_PAGE = 16

(QDEC_W_IN_NORM, QDEC_W_Q, QDEC_W_K, QDEC_W_V, QDEC_W_Q_NORM, QDEC_W_K_NORM, QDEC_W_O,
 QDEC_W_POST_NORM, QDEC_W_GATE, QDEC_W_UP, QDEC_W_DOWN, QDEC_W_PER_LAYER) = range(12)

EXPORTS = ("qdec_create", "qdec_destroy", "qdec_state_create", "qdec_state_destroy", "qdec_prefill",
           "qdec_decode_step", "qdec_decode_step_dev", "qdec_decode_greedy", "qdec_decode_batch", "qdec_sample",
           "qdec_sample_noalloc",
           "qdec_clone_state", "qdec_state_pos", "qdec_model_status", "qdec_last_error", "qdec_adaptor_create",
           "qdec_adaptor_run", "qdec_adaptor_destroy", "qdec_encoder_create", "qdec_encoder_rows",
           "qdec_frontend_run", "qdec_encoder_forward", "qdec_encoder_run", "qdec_encoder_destroy")

QDEC_SAMPLE_TOP_K_MAX = 128
QDEC_SAMPLE_NOALLOC_MAX_VOCAB = 153600


class QdecError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"qdec error {code}: {msg}")
        self.code = code


class qdec_config(ctypes.Structure):
    _fields_ = [("n_layer", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q_head", ctypes.c_int32),
                ("n_kv_head", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("weight_dtype", ctypes.c_int32), ("tied", ctypes.c_int32)]


class qdec_weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("layer", ctypes.POINTER(ctypes.c_void_p))]


class qdec_adaptor_config(ctypes.Structure):
    _fields_ = [("enc_dim", ctypes.c_int32), ("mid_dim", ctypes.c_int32), ("dim", ctypes.c_int32),
                ("ffn_dim", ctypes.c_int32), ("n_block", ctypes.c_int32), ("n_head", ctypes.c_int32),
                ("ln_eps", ctypes.c_float), ("weight_dtype", ctypes.c_int32)]


class qdec_adaptor_weights(ctypes.Structure):
    _fields_ = [("linear1_w", ctypes.c_void_p), ("linear1_b", ctypes.c_void_p), ("linear2_w", ctypes.c_void_p),
                ("linear2_b", ctypes.c_void_p), ("block", ctypes.POINTER(ctypes.c_void_p))]


# per-block tensor order of qdec_adaptor_weights.block
ADAPTOR_BLOCK_TENSORS = ("norm1.g", "norm1.b", "q.w", "q.b", "k.w", "k.b", "v.w", "v.b", "o.w", "o.b",
                         "norm2.g", "norm2.b", "fc1.w", "fc1.b", "fc2.w", "fc2.b")


class qdec_encoder_config(ctypes.Structure):
    _fields_ = [("n_mels", ctypes.c_int32), ("lfr_m", ctypes.c_int32), ("lfr_n", ctypes.c_int32),
                ("dim", ctypes.c_int32), ("n_head", ctypes.c_int32), ("ffn_dim", ctypes.c_int32),
                ("fsmn_kernel", ctypes.c_int32), ("n_main", ctypes.c_int32), ("n_tp", ctypes.c_int32),
                ("ln_eps", ctypes.c_float), ("weight_dtype", ctypes.c_int32)]


class qdec_encoder_weights(ctypes.Structure):
    _fields_ = [("block", ctypes.POINTER(ctypes.c_void_p)), ("after_norm_g", ctypes.c_void_p),
                ("after_norm_b", ctypes.c_void_p), ("tp_norm_g", ctypes.c_void_p), ("tp_norm_b", ctypes.c_void_p)]


# per-block tensor order of qdec_encoder_weights.block
ENCODER_BLOCK_TENSORS = ("norm1.g", "norm1.b", "q.w", "q.b", "k.w", "k.b", "v.w", "v.b", "fsmn.w", "o.w", "o.b",
                         "norm2.g", "norm2.b", "ffn1.w", "ffn1.b", "ffn2.w", "ffn2.b")


class qdec_sampling(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_k", ctypes.c_int32), ("top_p", ctypes.c_float),
                ("repetition_penalty", ctypes.c_float)]


_lib = None


def use_library(path: str) -> None:
    """Load the library from `path` instead of libqdec.so (the diagnostic
    build libqdec_trace.so); must run before the first call."""
    global LIB_PATH
    if _lib is not None:
        raise RuntimeError("the qdec library is already loaded")
    LIB_PATH = path


def lib() -> ctypes.CDLL:
    """Load libqdec.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} not built; run python -m qwen3_kv_cache_amd.build")
    # torch's ROCm wheel carries its own HIP runtime, loaded under the bare
    # name libamdhip64.so. Load it first: libqdec.so then binds to that same
    # runtime by soname, and the process holds a single HIP runtime (two
    # runtimes side by side do not share devices, streams or allocations).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    sig = {
        "qdec_create": (ctypes.c_int, [ctypes.POINTER(qdec_config), ctypes.POINTER(qdec_weights), vp,
                                       ctypes.POINTER(vp)]),
        "qdec_destroy": (ctypes.c_int, [vp]),
        "qdec_state_create": (ctypes.c_int, [vp, i32, ctypes.POINTER(vp)]),
        "qdec_state_destroy": (None, [vp]),
        "qdec_prefill": (ctypes.c_int, [vp, ctypes.POINTER(i32), i32, vp, i32, i32, vp, vp]),
        "qdec_decode_step": (ctypes.c_int, [vp, i32, i32, vp, vp]),
        "qdec_decode_step_dev": (ctypes.c_int, [vp, vp, i32, vp, vp]),
        "qdec_decode_greedy": (ctypes.c_int, [vp, vp, i32, i32, vp, vp]),
        "qdec_decode_batch": (ctypes.c_int, [ctypes.POINTER(vp), i32, ctypes.POINTER(i32), vp, vp]),
        "qdec_sample": (ctypes.c_int, [vp, vp, i32, ctypes.POINTER(qdec_sampling), vp, i32,
                                       ctypes.POINTER(ctypes.c_float), vp]),
        "qdec_sample_noalloc": (ctypes.c_int, [vp, vp, i32, ctypes.POINTER(qdec_sampling), vp, i32,
                                               ctypes.POINTER(ctypes.c_float), vp]),
        "qdec_clone_state": (ctypes.c_int, [vp, ctypes.POINTER(vp)]),
        "qdec_state_pos": (i32, [vp]),
        "qdec_model_status": (ctypes.c_int, [vp]),
        "qdec_last_error": (ctypes.c_char_p, []),
        "qdec_adaptor_create": (ctypes.c_int, [ctypes.POINTER(qdec_adaptor_config),
                                               ctypes.POINTER(qdec_adaptor_weights), vp, ctypes.POINTER(vp)]),
        "qdec_adaptor_run": (ctypes.c_int, [vp, vp, i32, vp]),
        "qdec_adaptor_destroy": (None, [vp]),
        "qdec_encoder_create": (ctypes.c_int, [ctypes.POINTER(qdec_encoder_config),
                                               ctypes.POINTER(qdec_encoder_weights), vp, ctypes.POINTER(vp)]),
        "qdec_encoder_rows": (i32, [vp, ctypes.c_int64]),
        "qdec_frontend_run": (ctypes.c_int, [vp, vp, ctypes.c_int64, vp]),
        "qdec_encoder_forward": (ctypes.c_int, [vp, vp, i32, vp]),
        "qdec_encoder_run": (ctypes.c_int, [vp, vp, ctypes.c_int64, vp]),
        "qdec_encoder_destroy": (None, [vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    if hasattr(L, "qdec_debug_trace"):  # diagnostic build only
        L.qdec_debug_trace.restype = ctypes.c_int
        L.qdec_debug_trace.argtypes = [ctypes.POINTER(ctypes.c_ulonglong), ctypes.c_int]
    _lib = L
    return L


def qdec_last_error() -> str:
    return lib().qdec_last_error().decode()


def _check(code: int) -> None:
    if code != QDEC_OK:
        raise QdecError(code, qdec_last_error())


def _ptr(p) -> Optional[int]:
    return None if p is None or p == 0 else int(p)


def qdec_create(cfg: qdec_config, weights: qdec_weights, stream: int = 0) -> int:
    out = ctypes.c_void_p()
    _check(lib().qdec_create(ctypes.byref(cfg), ctypes.byref(weights), _ptr(stream), ctypes.byref(out)))
    return out.value


def qdec_destroy(model: int) -> None:
    _check(lib().qdec_destroy(_ptr(model)))


def qdec_state_create(model: int, max_ctx: int) -> int:
    out = ctypes.c_void_p()
    _check(lib().qdec_state_create(_ptr(model), int(max_ctx), ctypes.byref(out)))
    return out.value


def qdec_state_destroy(state: int) -> None:
    lib().qdec_state_destroy(_ptr(state))


def qdec_prefill(state: int, ids_host, n_tokens: int, audio_dev, audio_begin: int, audio_len: int,
                 logits_dev=None, argmax_dev=None) -> None:
    ids = np.ascontiguousarray(ids_host, dtype=np.int32)
    if ids.size < n_tokens:
        raise ValueError("ids_host shorter than n_tokens")
    p = ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    _check(lib().qdec_prefill(_ptr(state), p, int(n_tokens), _ptr(audio_dev), int(audio_begin), int(audio_len),
                              _ptr(logits_dev), _ptr(argmax_dev)))


def qdec_decode_step(state: int, token: int, pos: int, logits_dev=None, argmax_dev=None) -> None:
    _check(lib().qdec_decode_step(_ptr(state), int(token), int(pos), _ptr(logits_dev), _ptr(argmax_dev)))


def qdec_decode_step_dev(state: int, token_dev, pos: int, logits_dev=None, argmax_dev=None) -> None:
    _check(lib().qdec_decode_step_dev(_ptr(state), _ptr(token_dev), int(pos), _ptr(logits_dev),
                                      _ptr(argmax_dev)))


def qdec_decode_greedy(state: int, token_dev, pos: int, n_steps: int, logits_dev=None, tokens_dev=None) -> None:
    _check(lib().qdec_decode_greedy(_ptr(state), _ptr(token_dev), int(pos), int(n_steps), _ptr(logits_dev),
                                    _ptr(tokens_dev)))


def qdec_decode_batch(states: Sequence[int], tokens_host, logits_dev=None, argmax_dev=None) -> None:
    n = len(states)
    arr = (ctypes.c_void_p * max(n, 1))(*[_ptr(s) for s in states])
    toks = np.ascontiguousarray(tokens_host, dtype=np.int32)
    if toks.size < n:
        raise ValueError("tokens_host shorter than the batch")
    _check(lib().qdec_decode_batch(arr, n, toks.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                   _ptr(logits_dev), _ptr(argmax_dev)))


def qdec_sample(model: int, logits_dev, n_rows: int, temperature: float, top_k: int, top_p: float,
                repetition_penalty: float, history_dev, history_len: int, uniforms_host, tokens_dev) -> None:
    p = qdec_sampling(float(temperature), int(top_k), float(top_p), float(repetition_penalty))
    u = np.ascontiguousarray(uniforms_host, dtype=np.float32)
    if u.size < n_rows:
        raise ValueError("uniforms_host shorter than n_rows")
    _check(lib().qdec_sample(_ptr(model), _ptr(logits_dev), int(n_rows), ctypes.byref(p), _ptr(history_dev),
                             int(history_len), u.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), _ptr(tokens_dev)))


def qdec_sample_noalloc(model: int, logits_dev, n_rows: int, temperature: float, top_k: int, top_p: float,
                        repetition_penalty: float, history_dev, history_len: int, uniforms_host, tokens_dev) -> None:
    p = qdec_sampling(float(temperature), int(top_k), float(top_p), float(repetition_penalty))
    u = np.ascontiguousarray(uniforms_host, dtype=np.float32)
    if u.size < n_rows:
        raise ValueError("uniforms_host shorter than n_rows")
    _check(lib().qdec_sample_noalloc(_ptr(model), _ptr(logits_dev), int(n_rows), ctypes.byref(p),
                                     _ptr(history_dev), int(history_len),
                                     u.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), _ptr(tokens_dev)))


def qdec_clone_state(src: int) -> int:
    out = ctypes.c_void_p()
    _check(lib().qdec_clone_state(_ptr(src), ctypes.byref(out)))
    return out.value


def qdec_adaptor_create(cfg: qdec_adaptor_config, weights: qdec_adaptor_weights, stream: int = 0) -> int:
    out = ctypes.c_void_p()
    _check(lib().qdec_adaptor_create(ctypes.byref(cfg), ctypes.byref(weights), _ptr(stream), ctypes.byref(out)))
    return out.value


def qdec_adaptor_run(adaptor: int, frames_dev, n_frames: int, out_dev) -> None:
    _check(lib().qdec_adaptor_run(_ptr(adaptor), _ptr(frames_dev), int(n_frames), _ptr(out_dev)))


def qdec_adaptor_destroy(adaptor: int) -> None:
    lib().qdec_adaptor_destroy(_ptr(adaptor))


def qdec_encoder_create(cfg: qdec_encoder_config, weights: qdec_encoder_weights, stream: int = 0) -> int:
    out = ctypes.c_void_p()
    _check(lib().qdec_encoder_create(ctypes.byref(cfg), ctypes.byref(weights), _ptr(stream), ctypes.byref(out)))
    return out.value


def qdec_encoder_rows(encoder: int, n_samples: int) -> int:
    return lib().qdec_encoder_rows(_ptr(encoder), int(n_samples))


def qdec_frontend_run(encoder: int, pcm_dev, n_samples: int, lfr_dev) -> None:
    _check(lib().qdec_frontend_run(_ptr(encoder), _ptr(pcm_dev), int(n_samples), _ptr(lfr_dev)))


def qdec_encoder_forward(encoder: int, lfr_dev, n_rows: int, out_dev) -> None:
    _check(lib().qdec_encoder_forward(_ptr(encoder), _ptr(lfr_dev), int(n_rows), _ptr(out_dev)))


def qdec_encoder_run(encoder: int, pcm_dev, n_samples: int, out_dev) -> None:
    _check(lib().qdec_encoder_run(_ptr(encoder), _ptr(pcm_dev), int(n_samples), _ptr(out_dev)))


def qdec_encoder_destroy(encoder: int) -> None:
    lib().qdec_encoder_destroy(_ptr(encoder))


def qdec_state_pos(state: int) -> int:
    return lib().qdec_state_pos(_ptr(state))


def qdec_model_status(model: int) -> None:
    """Raises QdecError(QDEC_E_DEVICE) if a device-side wait on this model has
    hit its time limit (check after synchronising the stream)."""
    _check(lib().qdec_model_status(_ptr(model)))


# ---------------------------------------------------------------- helpers

def make_config(hidden, n_layer, n_q_head, n_kv_head, head_dim, ffn, vocab, rms_eps=1e-6, rope_theta=1e6,
                bf16=True, tied=1, weight_dtype=None) -> qdec_config:
    """weight_dtype (QDEC_F32, QDEC_BF16, QDEC_Q8_0) overrides `bf16` when given."""
    if weight_dtype is None:
        weight_dtype = QDEC_BF16 if bf16 else QDEC_F32
    return qdec_config(n_layer, hidden, n_q_head, n_kv_head, head_dim, ffn, vocab, rms_eps, rope_theta,
                       weight_dtype, tied)


class WeightTable:
    """qdec_weights built from device addresses; keeps the host pointer table
    alive. `layer_ptrs[i][t]` is layer i's tensor t (QDEC_W_* order)."""

    def __init__(self, embed: int, final_norm: int, layer_ptrs: Sequence[Sequence[int]]):
        flat = [int(p) for row in layer_ptrs for p in row]
        self._arr = (ctypes.c_void_p * max(len(flat), 1))(*flat)
        self.c = qdec_weights(int(embed), int(final_norm),
                              ctypes.cast(self._arr, ctypes.POINTER(ctypes.c_void_p)))
