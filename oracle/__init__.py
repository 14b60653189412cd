"""CPU float64 oracle of the decoder-layer prefill (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  It shares no code with the HIP library.
"""
from .layer import (apply_rope, argmax_rows, as_dense, cache_store, causal_gqa_attention, decode_sign1,
                    lm_head_logits, prefill_chunk, prefill_layer, qkv_rows, rms_norm,
                    rope_inv_freq, silu, verify_tail)

__all__ = ["apply_rope", "argmax_rows", "as_dense", "cache_store", "causal_gqa_attention", "decode_sign1",
           "lm_head_logits", "prefill_chunk", "prefill_layer", "qkv_rows", "rms_norm",
           "rope_inv_freq", "silu", "verify_tail"]
