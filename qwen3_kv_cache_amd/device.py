"""Device-memory plumbing around the C ABI (PyTorch allocates, qdec computes).

``Model`` uploads a weight mapping to the GPU with torch and creates a qdec
model on the current torch stream. The mapping uses the names "embed",
"final_norm" and "L{i}.{in_norm,wq,wk,wv,q_norm,k_norm,wo,post_norm,w_gate,
w_up,w_down}"; bf16 weights are given as uint16 bit patterns.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from . import qdec

LAYER_TENSORS = ("in_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "post_norm", "w_gate", "w_up", "w_down")


def _torch():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("qdec needs a ROCm GPU; none is visible")
    return torch


class Model:
    def __init__(self, shape, arrays: Dict[str, np.ndarray], bf16: bool, device: str = "cuda:0"):
        torch = _torch()
        self.shape = shape
        self.device = torch.device(device)
        self.bf16 = bf16
        self.tensors = {}
        for name, a in arrays.items():
            if bf16:
                t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(self.device).view(torch.bfloat16)
            else:
                t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(self.device)
            self.tensors[name] = t
        layer_ptrs = [[self.tensors[f"L{i}.{t}"].data_ptr() for t in LAYER_TENSORS] for i in range(shape.n_layer)]
        self.table = qdec.WeightTable(self.tensors["embed"].data_ptr(), self.tensors["final_norm"].data_ptr(),
                                      layer_ptrs)
        self.cfg = qdec.make_config(shape.hidden, shape.n_layer, shape.n_q_head, shape.n_kv_head, shape.head_dim,
                                    shape.ffn, shape.vocab, shape.rms_eps, shape.rope_theta, bf16=bf16)
        self.stream = torch.cuda.current_stream(self.device).cuda_stream
        self.handle = qdec.qdec_create(self.cfg, self.table.c, self.stream)
        # packed copies now live inside the library; keep only the tied embedding
        for name in list(self.tensors):
            if name != "embed":
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
