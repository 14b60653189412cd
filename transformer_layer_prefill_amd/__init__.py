"""MI355X (gfx950) transformer-layer prefill: HIP kernels behind a C ABI.

The Python side is a thin binding of ``libtlp.so`` (include/tlp.h); torch
supplies device memory and streams.  Build the library with
``transformer_layer_prefill_amd.build.build()``.
"""
from ._lib import (EXPORTS, KERNELS, LIB_PATH, TLP_BF16, TLP_ERR_HIP, TLP_ERR_NULL,
                   TLP_ERR_POSITION, TLP_ERR_SHAPE, TLP_ERR_UNSUPPORTED, TLP_ERR_WORKSPACE,
                   TLP_F32, TLP_KV_ACT, TLP_KV_F16, TLP_OK, TLP_W_DENSE, TLP_W_SIGN1_G128, WS_ACT, WS_ATTN, WS_COUNT,
                   WS_HEAD, WS_PART, WS_QKV, WS_RES, WS_XN, Config, LayerWeights, TlpError,
                   Pipeline, Weight, argmax_rows, lib, make_config, prefill_chunk, prefill_layer,
                   prefill_layer_noalloc, NOALLOC_SCRATCH_BYTES,
                   profile_begin, profile_end, rope_table, verify_tail, verify_workspace_bytes,
                   workspace_bytes, workspace_layout)

__all__ = ["EXPORTS", "KERNELS", "LIB_PATH", "profile_begin", "profile_end", "Config", "Pipeline",
           "LayerWeights", "TlpError", "Weight", "lib", "make_config", "prefill_chunk",
           "prefill_layer", "prefill_layer_noalloc", "NOALLOC_SCRATCH_BYTES", "rope_table", "workspace_bytes", "workspace_layout", "argmax_rows",
           "verify_tail", "verify_workspace_bytes", "TLP_OK", "TLP_ERR_NULL", "TLP_ERR_SHAPE",
           "TLP_ERR_POSITION", "TLP_ERR_UNSUPPORTED", "TLP_ERR_WORKSPACE", "TLP_ERR_HIP",
           "TLP_F32", "TLP_BF16", "TLP_KV_ACT", "TLP_KV_F16", "TLP_W_DENSE", "TLP_W_SIGN1_G128", "WS_RES", "WS_XN", "WS_QKV",
           "WS_ATTN", "WS_ACT", "WS_HEAD", "WS_PART", "WS_COUNT"]
