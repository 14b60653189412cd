"""Device-memory plumbing around the C ABI: upload storage-format arrays as
torch tensors and fill the ctypes weight structs with their addresses.

torch only provides device memory and streams here; nothing is computed.
"""
from __future__ import annotations

import numpy as np

from . import _lib


def to_device(a: np.ndarray, device="cuda"):
    """numpy storage array -> torch device tensor with the same bytes.

    uint16 arrays are bf16 bit patterns and come back as torch.bfloat16;
    uint32 (1-bit sign words) come back as int32; float16/float32 as is.
    """
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).to(device)
    if a.dtype in (np.float16, np.float32):
        return torch.from_numpy(a).to(device)
    raise TypeError(f"unsupported storage dtype {a.dtype}")


def to_host(t) -> np.ndarray:
    """torch tensor -> numpy storage array (bf16 -> uint16 bit patterns)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.int32:
        return t.numpy().view(np.uint32)
    return t.numpy()


def config_of(shape) -> _lib.Config:
    """C config for a layer shape (anything with the fields of synth.Shape)."""
    return _lib.make_config(shape.hidden, shape.inter, shape.nq, shape.nkv, shape.head_dim,
                            shape.max_seq, shape.n_layers, shape.eps, shape.qk_norm,
                            _lib.TLP_F32 if shape.dtype == "f32" else _lib.TLP_BF16,
                            _lib.TLP_W_SIGN1_G128 if shape.wformat == "sign1"
                            else _lib.TLP_W_DENSE,
                            _lib.TLP_KV_F16 if getattr(shape, "kv", "act") == "f16"
                            else _lib.TLP_KV_ACT)


class DeviceLayer:
    """One layer's weights resident on the device plus their C struct."""

    PROJ = ("w_qkv", "w_o", "w_gate_up", "w_down")
    GAIN = ("attn_norm", "q_norm", "k_norm", "ffn_norm")

    def __init__(self, w: dict, device="cuda"):
        self.t = {}
        for k, v in w.items():
            if isinstance(v, dict):
                self.t[k] = (to_device(v["bits"], device), to_device(v["scales"], device))
            else:
                self.t[k] = (to_device(v, device), None)
        s = _lib.LayerWeights()
        for k in self.GAIN:
            setattr(s, k, self.t[k][0].data_ptr())
        for k in self.PROJ:
            data, scales = self.t[k]
            setattr(s, k, _lib.Weight(data.data_ptr(), scales.data_ptr() if scales is not None
                                      else None))
        self.struct = s
