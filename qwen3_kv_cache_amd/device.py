"""Device-memory plumbing around the C ABI (PyTorch allocates, qdec computes).

``Model`` uploads a weight mapping to the GPU with torch and creates a qdec
model on the current torch stream. The mapping uses the names "embed",
"final_norm" and "L{i}.{in_norm,wq,wk,wv,q_norm,k_norm,wo,post_norm,w_gate,
w_up,w_down}"; bf16 weights are given as uint16 bit patterns. With q8=True
the matrices and the embedding are uint8 arrays of Q8_0 blocks (one row of
in / 32 blocks of 34 bytes per matrix row) and the norm gains float32.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from . import qdec

LAYER_TENSORS = ("in_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "post_norm", "w_gate", "w_up", "w_down")
NORM_TENSORS = ("in_norm", "q_norm", "k_norm", "post_norm", "final_norm")


def _torch():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("qdec needs a ROCm GPU; none is visible")
    return torch


class Model:
    def __init__(self, shape, arrays: Dict[str, np.ndarray], bf16: bool, device: str = "cuda:0", q8: bool = False):
        torch = _torch()
        self.shape = shape
        self.device = torch.device(device)
        self.bf16 = bf16 and not q8
        self.q8 = q8
        self.tensors = {}
        for name, a in arrays.items():
            if q8:
                is_norm = name.split(".")[-1] in NORM_TENSORS
                a = np.ascontiguousarray(a, dtype=np.float32 if is_norm else np.uint8)
                t = torch.from_numpy(a).to(self.device)
            elif bf16:
                t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(self.device).view(torch.bfloat16)
            else:
                t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(self.device)
            self.tensors[name] = t
        layer_ptrs = [[self.tensors[f"L{i}.{t}"].data_ptr() for t in LAYER_TENSORS] for i in range(shape.n_layer)]
        self.table = qdec.WeightTable(self.tensors["embed"].data_ptr(), self.tensors["final_norm"].data_ptr(),
                                      layer_ptrs)
        dtype = qdec.QDEC_Q8_0 if q8 else (qdec.QDEC_BF16 if bf16 else qdec.QDEC_F32)
        self.cfg = qdec.make_config(shape.hidden, shape.n_layer, shape.n_q_head, shape.n_kv_head, shape.head_dim,
                                    shape.ffn, shape.vocab, shape.rms_eps, shape.rope_theta, weight_dtype=dtype)
        self.stream = torch.cuda.current_stream(self.device).cuda_stream
        self.handle = qdec.qdec_create(self.cfg, self.table.c, self.stream)
        # packed copies now live inside the library; keep only a borrowed
        # embedding (Q8_0 embeddings are unpacked into the library's copies)
        for name in list(self.tensors):
            if name != "embed" or q8:
                del self.tensors[name]
        torch.cuda.synchronize(self.device)

    def close(self) -> None:
        if self.handle:
            qdec.qdec_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Adaptor:
    """The audio adaptor on the GPU: ``bits`` maps the parameter names
    ("linear1.w", "linear1.b", "linear2.w", "linear2.b", "blocks.{i}.<t>" for
    t in qdec.ADAPTOR_BLOCK_TENSORS) to bf16 bit patterns (uint16)."""

    def __init__(self, shape, bits: Dict[str, np.ndarray], ln_eps: float = 1e-12, device: str = "cuda:0"):
        torch = _torch()
        self.shape = shape
        self.device = torch.device(device)
        self.tensors = {name: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(self.device)
                        for name, a in bits.items()}
        blocks = [self.tensors[f"blocks.{i}.{t}"].data_ptr() for i in range(shape.n_block)
                  for t in qdec.ADAPTOR_BLOCK_TENSORS]
        self._block_arr = (qdec.ctypes.c_void_p * len(blocks))(*blocks)
        w = qdec.qdec_adaptor_weights(self.tensors["linear1.w"].data_ptr(), self.tensors["linear1.b"].data_ptr(),
                                      self.tensors["linear2.w"].data_ptr(), self.tensors["linear2.b"].data_ptr(),
                                      qdec.ctypes.cast(self._block_arr, qdec.ctypes.POINTER(qdec.ctypes.c_void_p)))
        self.cfg = qdec.qdec_adaptor_config(shape.enc_dim, shape.mid_dim, shape.dim, shape.ffn_dim, shape.n_block,
                                            shape.n_head, ln_eps, qdec.QDEC_BF16)
        self.stream = torch.cuda.current_stream(self.device).cuda_stream
        self.handle = qdec.qdec_adaptor_create(self.cfg, w, self.stream)
        torch.cuda.synchronize(self.device)

    def run(self, frames, out=None):
        """frames: fp32 device tensor [T, enc_dim]; returns [T, dim] fp32."""
        torch = _torch()
        T = frames.shape[0]
        if out is None:
            out = torch.empty((T, self.shape.dim), dtype=torch.float32, device=self.device)
        qdec.qdec_adaptor_run(self.handle, frames.data_ptr(), T, out.data_ptr())
        return out

    def close(self) -> None:
        if self.handle:
            qdec.qdec_adaptor_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Encoder:
    """The audio frontend and SAN-M encoder on the GPU: ``bits`` maps the
    parameter names ("{block}<t>" for each block prefix of
    shape.block_names() and t in qdec.ENCODER_BLOCK_TENSORS, "after_norm.g",
    "after_norm.b", "tp_norm.g", "tp_norm.b") to bf16 bit patterns (uint16)."""

    def __init__(self, shape, bits: Dict[str, np.ndarray], ln_eps: float = 1e-12, n_mels: int = 80,
                 lfr_m: int = 7, lfr_n: int = 6, device: str = "cuda:0"):
        torch = _torch()
        self.shape = shape
        self.device = torch.device(device)
        self.tensors = {name: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(self.device)
                        for name, a in bits.items()}
        blocks = [self.tensors[pre + t].data_ptr() for pre in shape.block_names()
                  for t in qdec.ENCODER_BLOCK_TENSORS]
        self._block_arr = (qdec.ctypes.c_void_p * len(blocks))(*blocks)
        w = qdec.qdec_encoder_weights(qdec.ctypes.cast(self._block_arr, qdec.ctypes.POINTER(qdec.ctypes.c_void_p)),
                                      self.tensors["after_norm.g"].data_ptr(), self.tensors["after_norm.b"].data_ptr(),
                                      self.tensors["tp_norm.g"].data_ptr(), self.tensors["tp_norm.b"].data_ptr())
        self.cfg = qdec.qdec_encoder_config(n_mels, lfr_m, lfr_n, shape.dim, shape.n_head, shape.ffn_dim,
                                            shape.kernel, shape.n_main, shape.n_tp, ln_eps, qdec.QDEC_BF16)
        self.in_dim = n_mels * lfr_m
        self.stream = torch.cuda.current_stream(self.device).cuda_stream
        self.handle = qdec.qdec_encoder_create(self.cfg, w, self.stream)
        # q/k/v, taps and vectors are copied; o, ffn1 and ffn2 stay borrowed
        keep = ("o.w", "ffn1.w", "ffn2.w")
        for name in list(self.tensors):
            if not name.endswith(keep):
                del self.tensors[name]
        torch.cuda.synchronize(self.device)

    def rows(self, n_samples: int) -> int:
        return qdec.qdec_encoder_rows(self.handle, n_samples)

    def frontend(self, pcm):
        """pcm: fp32 device tensor [n]; returns the LFR rows [rows, 560] fp32."""
        torch = _torch()
        out = torch.empty((self.rows(pcm.shape[0]), self.in_dim), dtype=torch.float32, device=self.device)
        qdec.qdec_frontend_run(self.handle, pcm.data_ptr(), pcm.shape[0], out.data_ptr())
        return out

    def forward(self, lfr):
        """lfr: fp32 device tensor [rows, 560]; returns the encoder frames [rows, dim]."""
        torch = _torch()
        out = torch.empty((lfr.shape[0], self.shape.dim), dtype=torch.float32, device=self.device)
        qdec.qdec_encoder_forward(self.handle, lfr.data_ptr(), lfr.shape[0], out.data_ptr())
        return out

    def run(self, pcm, out=None):
        """pcm: fp32 device tensor [n]; returns the encoder frames [rows, dim]."""
        torch = _torch()
        if out is None:
            out = torch.empty((self.rows(pcm.shape[0]), self.shape.dim), dtype=torch.float32, device=self.device)
        qdec.qdec_encoder_run(self.handle, pcm.data_ptr(), pcm.shape[0], out.data_ptr())
        return out

    def close(self) -> None:
        if self.handle:
            qdec.qdec_encoder_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
