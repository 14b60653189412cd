"""ctypes binding of ``libtlp.so`` (include/tlp.h): argument marshalling only.

Every computation happens in the HIP library.  Functions take torch device
tensors (or raw integer device addresses) and the current torch stream; when
the library is missing this module raises instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtlp.so")

TLP_OK, TLP_ERR_NULL, TLP_ERR_SHAPE, TLP_ERR_POSITION = 0, 1, 2, 3
TLP_ERR_UNSUPPORTED, TLP_ERR_WORKSPACE, TLP_ERR_HIP = 4, 5, 6
TLP_F32, TLP_BF16 = 0, 1
TLP_W_DENSE, TLP_W_SIGN1_G128 = 0, 1
TLP_KV_ACT, TLP_KV_F16 = 0, 1
WS_RES, WS_XN, WS_QKV, WS_ATTN, WS_ACT, WS_HEAD, WS_PART, WS_COUNT = range(8)
NOALLOC_SCRATCH_BYTES = 64 << 20   # TLP_NOALLOC_SCRATCH_BYTES

EXPORTS = ("tlp_workspace_bytes", "tlp_workspace_layout", "tlp_rope_table",
           "tlp_prefill_layer", "tlp_prefill_layer_noalloc", "tlp_prefill_chunk", "tlp_argmax_rows",
           "tlp_verify_workspace_bytes", "tlp_verify_tail", "tlp_pipeline_create",
           "tlp_pipeline_destroy", "tlp_profile_begin",
           "tlp_profile_end", "tlp_status_string", "tlp_last_error")
KERNELS = ("attn_norm", "qkv_gemm", "qk_rope_kv", "attention", "o_gemm", "ffn_norm",
           "gate_up_gemm", "down_gemm", "final_norm", "lm_head", "out_rows", "swiglu",
           "argmax")


class TlpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"tlp status {status}: {message}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_seq", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("qk_norm", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("wformat", ctypes.c_int32), ("kv_format", ctypes.c_int32)]


class Weight(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("attn_norm", ctypes.c_void_p), ("w_qkv", Weight), ("q_norm", ctypes.c_void_p),
                ("k_norm", ctypes.c_void_p), ("w_o", Weight), ("ffn_norm", ctypes.c_void_p),
                ("w_gate_up", Weight), ("w_down", Weight)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        cfgp = ctypes.POINTER(Config)
        L.tlp_workspace_bytes.argtypes = [cfgp, i32]
        L.tlp_workspace_bytes.restype = sz
        L.tlp_workspace_layout.argtypes = [cfgp, i32, ctypes.POINTER(sz)]
        L.tlp_workspace_layout.restype = ctypes.c_int
        L.tlp_rope_table.argtypes = [ctypes.c_double, i32, i32, vp, vp]
        L.tlp_rope_table.restype = ctypes.c_int
        L.tlp_prefill_layer.argtypes = [cfgp, ctypes.POINTER(LayerWeights), i32, vp, i32, i32,
                                        vp, vp, vp, vp, vp, sz, vp]
        L.tlp_prefill_layer.restype = ctypes.c_int
        L.tlp_prefill_layer_noalloc.argtypes = [cfgp, ctypes.POINTER(LayerWeights), i32, vp, i32,
                                                i32, vp, vp, vp, vp, vp]
        L.tlp_prefill_layer_noalloc.restype = ctypes.c_int
        L.tlp_prefill_chunk.argtypes = [cfgp, ctypes.POINTER(LayerWeights), vp, i32, i32, i32,
                                        vp, vp, vp, vp, vp, vp, i32, ctypes.c_float, vp, vp, sz,
                                        vp, vp]
        L.tlp_pipeline_create.argtypes = [i32, ctypes.POINTER(vp)]
        L.tlp_pipeline_create.restype = ctypes.c_int
        L.tlp_pipeline_destroy.argtypes = [vp]
        L.tlp_pipeline_destroy.restype = ctypes.c_int
        L.tlp_prefill_chunk.restype = ctypes.c_int
        L.tlp_argmax_rows.argtypes = [vp, i32, i32, ctypes.c_int64, vp, vp]
        L.tlp_argmax_rows.restype = ctypes.c_int
        L.tlp_verify_workspace_bytes.argtypes = [cfgp, i32]
        L.tlp_verify_workspace_bytes.restype = sz
        L.tlp_verify_tail.argtypes = [cfgp, vp, i32, vp, vp, i32, ctypes.c_float, vp, vp, vp,
                                      sz, vp]
        L.tlp_verify_tail.restype = ctypes.c_int
        L.tlp_profile_begin.argtypes = [i32]
        L.tlp_profile_begin.restype = ctypes.c_int
        L.tlp_profile_end.argtypes = [vp, vp, vp]
        L.tlp_profile_end.restype = ctypes.c_int
        L.tlp_status_string.argtypes = [ctypes.c_int]
        L.tlp_status_string.restype = ctypes.c_char_p
        L.tlp_last_error.argtypes = []
        L.tlp_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != TLP_OK:
        raise TlpError(status, lib().tlp_last_error().decode())


def _ptr(x) -> int | None:
    """Device address of a torch tensor (or an int / None passed through)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_config(hidden, intermediate, n_q_heads, n_kv_heads, head_dim, max_seq, n_layers,
                rms_eps, qk_norm, dtype, wformat=TLP_W_DENSE, kv_format=TLP_KV_ACT) -> Config:
    return Config(hidden, intermediate, n_q_heads, n_kv_heads, head_dim, max_seq, n_layers,
                  rms_eps, int(bool(qk_norm)), dtype, wformat, kv_format)


def workspace_bytes(cfg: Config, max_tokens: int) -> int:
    return int(lib().tlp_workspace_bytes(ctypes.byref(cfg), max_tokens))


def workspace_layout(cfg: Config, max_tokens: int) -> list:
    offs = (ctypes.c_size_t * WS_COUNT)()
    _check(lib().tlp_workspace_layout(ctypes.byref(cfg), max_tokens, offs))
    return list(offs)


def rope_table(theta: float, head_dim: int, n_pos: int):
    """Host fp32 cos/sin tables [n_pos][head_dim/2] built by the library."""
    half = max(head_dim // 2, 1)
    cos = np.empty((max(n_pos, 1), half), dtype=np.float32)
    sin = np.empty_like(cos)
    _check(lib().tlp_rope_table(theta, head_dim, n_pos, cos.ctypes.data, sin.ctypes.data))
    return cos, sin


def prefill_layer(cfg: Config, weights: LayerWeights, layer: int, hidden, n_tokens: int,
                  start_position: int, k_cache, v_cache, rope_cos, rope_sin, workspace,
                  workspace_bytes: int | None = None, stream=None) -> None:
    wsb = workspace_bytes if workspace_bytes is not None else \
        workspace.numel() * workspace.element_size()
    _check(lib().tlp_prefill_layer(ctypes.byref(cfg), ctypes.byref(weights), layer,
                                   _ptr(hidden), n_tokens, start_position, _ptr(k_cache),
                                   _ptr(v_cache), _ptr(rope_cos), _ptr(rope_sin),
                                   _ptr(workspace), wsb, _stream(stream)))


def prefill_layer_noalloc(cfg: Config, weights: LayerWeights, layer: int, hidden, n_tokens: int,
                          start_position: int, k_cache, v_cache, rope_cos, rope_sin,
                          stream=None) -> None:
    """tlp_prefill_layer with the library's static per-GPU scratch as workspace."""
    _check(lib().tlp_prefill_layer_noalloc(ctypes.byref(cfg), ctypes.byref(weights), layer,
                                           _ptr(hidden), n_tokens, start_position,
                                           _ptr(k_cache), _ptr(v_cache), _ptr(rope_cos),
                                           _ptr(rope_sin), _stream(stream)))


class Pipeline:
    """A tlp_pipeline: the second stream and events that let prefill_chunk keep
    two micro-batches in flight.  Made on the current device; released by
    close() or when garbage-collected."""

    def __init__(self, max_layers: int):
        h = ctypes.c_void_p()
        _check(lib().tlp_pipeline_create(max_layers, ctypes.byref(h)))
        self.handle = h.value
        self.max_layers = max_layers

    def close(self) -> None:
        if self.handle:
            h, self.handle = self.handle, None
            _check(lib().tlp_pipeline_destroy(h))

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def prefill_chunk(cfg: Config, layers, hidden, n_tokens: int, start_position: int,
                  micro_batch: int, k_cache, v_cache, rope_cos, rope_sin, workspace,
                  final_norm=None, lm_head=None, vocab: int = 0, final_eps: float = 0.0,
                  logits=None, workspace_bytes: int | None = None, pipeline=None,
                  stream=None) -> None:
    arr = (LayerWeights * len(layers))(*layers)
    wsb = workspace_bytes if workspace_bytes is not None else \
        workspace.numel() * workspace.element_size()
    pipe = pipeline.handle if isinstance(pipeline, Pipeline) else pipeline
    _check(lib().tlp_prefill_chunk(ctypes.byref(cfg), arr, _ptr(hidden), n_tokens,
                                   start_position, micro_batch, _ptr(k_cache), _ptr(v_cache),
                                   _ptr(rope_cos), _ptr(rope_sin), _ptr(final_norm),
                                   _ptr(lm_head), vocab, final_eps, _ptr(logits),
                                   _ptr(workspace), wsb, pipe, _stream(stream)))


def argmax_rows(logits, rows: int, vocab: int, ld: int, token_ids, stream=None) -> None:
    _check(lib().tlp_argmax_rows(_ptr(logits), rows, vocab, ld, _ptr(token_ids),
                                 _stream(stream)))


def verify_workspace_bytes(cfg: Config, n_rows: int) -> int:
    return int(lib().tlp_verify_workspace_bytes(ctypes.byref(cfg), n_rows))


def verify_tail(cfg: Config, hidden, n_rows: int, final_norm, lm_head, vocab: int,
                final_eps: float, logits, token_ids, workspace,
                workspace_bytes: int | None = None, stream=None) -> None:
    wsb = workspace_bytes if workspace_bytes is not None else \
        workspace.numel() * workspace.element_size()
    _check(lib().tlp_verify_tail(ctypes.byref(cfg), _ptr(hidden), n_rows, _ptr(final_norm),
                                 _ptr(lm_head), vocab, final_eps, _ptr(logits),
                                 _ptr(token_ids), _ptr(workspace), wsb, _stream(stream)))


def profile_begin(max_launches: int = 8192) -> None:
    _check(lib().tlp_profile_begin(max_launches))


def profile_end() -> dict:
    """{kernel name: (launches, total milliseconds)} since profile_begin();
    launches past its capacity are not timed (key "not_timed")."""
    ms = np.zeros(len(KERNELS), dtype=np.float64)
    n = np.zeros(len(KERNELS), dtype=np.int32)
    dropped = ctypes.c_int32(0)
    _check(lib().tlp_profile_end(ms.ctypes.data, n.ctypes.data, ctypes.byref(dropped)))
    out = {k: (int(n[i]), float(ms[i])) for i, k in enumerate(KERNELS)}
    out["not_timed"] = (int(dropped.value), 0.0)
    return out
