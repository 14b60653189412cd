"""CPU float64 oracle of the batched decoder-layer prefill.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The HIP
library never does, and this module imports nothing from it.

What is computed, and where the pages define it.  The pages are three
Metal/Rust sources on docs.rs:

* [prefill page]  oxibonsai-kernels 0.1.1, ``gpu_backend/metal_prefill.rs``
* [layer page]    oxibonsai-kernels 0.1.0, ``gpu_backend/metal_full_layer.rs``
* [chunk page]    turbospark-runtime 0.3.0, ``families/llama/prefill.rs``

The layer is ``encode_layer_prefill`` on the prefill page (its steps 1-7,
with step 3's per-token attention sub-steps a-e); the chunk driver is
``prefill_chunk_real_llama_dense`` on the chunk page; the last-token head is
the "Tail" block of ``encode_full_forward_prefill`` on the prefill page.  The
kernel bodies are not on the pages, so where they leave a formula open this
file takes the plain reading and says so in the function's docstring.

Everything is float64 with no rounding anywhere; inputs arrive already widened
exactly from their storage formats.  Matrix products use ``numpy @`` as a
library step; nothing is blocked, fused or reordered beyond the definitions.
"""
from __future__ import annotations

import math

import numpy as np

SIGN1_GROUP = 128


# ---------------------------------------------------------------------------
# elementary operations
# ---------------------------------------------------------------------------

def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: ``gain * x / sqrt(mean(x^2) + eps)``.

    Prefill page, ``encode_layer_prefill`` steps 1 and 5 (batched RMSNorm of
    every token's row with a weight vector and ``eps``); the same operation
    is applied per head for QK-norm (step 3a).  Reading: mean over the row,
    eps inside the square root, the gain multiplies directly (no ``1 + g``).
    """
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return gain * (x / np.sqrt(ms + eps))


def rope_inv_freq(theta: float, head_dim: int) -> np.ndarray:
    """Per-pair frequencies ``theta^(-2i/hd)`` for i < hd/2.

    The pages build the cos/sin tables on the host (prefill page,
    ``encode_full_forward_prefill`` arguments ``cos_table``/``sin_table`` of
    ``half_dim`` entries per position); the frequency law is the standard
    rotary one, with no extra frequency scaling.
    """
    i = np.arange(head_dim // 2, dtype=np.float64)
    return theta ** (-2.0 * i / head_dim)


def apply_rope(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding of ``x[n, heads, hd]`` at absolute ``positions[n]``.

    Prefill page, ``encode_layer_prefill`` step 3c (fused QK RoPE with a
    ``half_dim``-wide cos/sin row per token).  Reading: rotate-half pairing,
    element i is paired with element i + hd/2 and the pair is rotated by the
    angle ``p * theta^(-2i/hd)``.
    """
    hd = x.shape[-1]
    half = hd // 2
    ang = np.outer(positions.astype(np.float64), rope_inv_freq(theta, hd))   # [n, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU ``z / (1 + exp(-z))``, the SwiGLU gate (chunk page, ``use_silu``)."""
    return z / (1.0 + np.exp(-z))


def decode_sign1(bits: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Dense float64 ``[N][K]`` from 1-bit signs and per-128-column scales.

    The 1-bit weight format itself is not on the pages (the layer page only
    says the 1-bit blocks are re-laid out structure-of-arrays for the GPU);
    this library fixes it: bit b of word w is column 32w+b, least significant
    bit first; 1 means +1 and 0 means -1; ``scales[n][g]`` multiplies columns
    128g .. 128g+127 of row n.  Decoded row block by row block to bound memory.
    """
    n, kw = bits.shape
    k = kw * 32
    out = np.empty((n, k), dtype=np.float64)
    shifts = np.arange(32, dtype=np.uint32)
    for r0 in range(0, n, 1024):
        b = bits[r0:r0 + 1024]
        one = ((b[:, :, None] >> shifts) & np.uint32(1)).reshape(b.shape[0], k)
        sign = np.where(one == 1, 1.0, -1.0)
        out[r0:r0 + 1024] = sign * np.repeat(scales[r0:r0 + 1024].astype(np.float64),
                                             SIGN1_GROUP, axis=1)
    return out


def as_dense(w) -> np.ndarray:
    """A projection weight as float64 ``[N][K]`` (dense array or (bits, scales))."""
    if isinstance(w, tuple):
        return decode_sign1(*w)
    return np.asarray(w, dtype=np.float64)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def causal_gqa_attention(q: np.ndarray, k_layer: np.ndarray, v_layer: np.ndarray,
                         positions: np.ndarray) -> np.ndarray:
    """Causal grouped-query attention of query rows against one layer's cache.

    ``q[r, nq, hd]`` are roped queries at absolute ``positions[r]``;
    ``k_layer``/``v_layer`` are ``[nkv][max_seq][hd]``.  Prefill page,
    ``encode_layer_prefill`` step 3e: scores ``q_h . K[u] / sqrt(hd)`` over
    ``seq_len = pos + 1`` keys (key u visible iff u <= pos), a softmax over
    them, then the softmax-weighted sum of V; query head h reads kv head
    ``h // (nq / nkv)`` (``heads_per_group``).  Returns ``[r, nq, hd]``.
    """
    r, nq, hd = q.shape
    nkv = k_layer.shape[0]
    group = nq // nkv
    scale = 1.0 / math.sqrt(hd)
    n_keys = int(positions.max()) + 1
    hidden_key = np.arange(n_keys)[None, :] > positions[:, None]       # [r, n_keys]
    out = np.empty((r, nq, hd), dtype=np.float64)
    for h in range(nq):
        j = h // group
        scores = (q[:, h, :] @ k_layer[j, :n_keys].T) * scale
        scores[hidden_key] = -np.inf
        scores = scores - scores.max(axis=1, keepdims=True)
        w = np.exp(scores)
        w = w / w.sum(axis=1, keepdims=True)
        out[:, h, :] = w @ v_layer[j, :n_keys]
    return out


# ---------------------------------------------------------------------------
# the layer and the chunk driver
# ---------------------------------------------------------------------------

def qkv_rows(shape, w: dict, x: np.ndarray, positions: np.ndarray):
    """Steps 1-3c for every token: RMSNorm, fused QKV, optional QK-norm, RoPE.

    Prefill page, ``encode_layer_prefill`` steps 1, 2, 3a-3c.  The fused QKV
    weight has the Q rows, then K, then V (the per-token byte offsets in step
    3a).  QK-norm uses one ``[hd]`` gain per side shared by all heads and the
    layer eps (layer page: q/k norm weights of head_dim floats).  V is neither
    normed nor rotated.  Returns roped q ``[n,nq,hd]``, roped k and raw v
    ``[n,nkv,hd]``.
    """
    n = x.shape[0]
    nq, nkv, hd = shape.nq, shape.nkv, shape.head_dim
    xn = rms_norm(x, w["attn_norm"], shape.eps)
    qkv = xn @ as_dense(w["w_qkv"]).T
    q = qkv[:, :nq * hd].reshape(n, nq, hd)
    k = qkv[:, nq * hd:(nq + nkv) * hd].reshape(n, nkv, hd)
    v = qkv[:, (nq + nkv) * hd:].reshape(n, nkv, hd)
    if shape.qk_norm:
        q = rms_norm(q, w["q_norm"], shape.eps)
        k = rms_norm(k, w["k_norm"], shape.eps)
    q = apply_rope(q, positions, shape.theta)
    k = apply_rope(k, positions, shape.theta)
    return q, k, v


def cache_store(shape, kv: np.ndarray) -> np.ndarray:
    """Values as a KV cache of the shape's format holds them.

    The layer page's ``GpuKvCache`` and the chunk page's attention keep K and
    V in f16; with that format (``shape.kv == "f16"``) a stored value is the
    nearest IEEE half (ties to even, numpy's conversion), so later attention
    reads the rounded value.  Otherwise the cache is exact here.
    """
    if getattr(shape, "kv", "act") == "f16":
        with np.errstate(over="ignore"):    # beyond the half range is +-inf by definition
            return np.asarray(kv, dtype=np.float64).astype(np.float16).astype(np.float64)
    return kv


def prefill_layer(shape, w: dict, layer: int, x: np.ndarray, start: int,
                  k_cache: np.ndarray, v_cache: np.ndarray,
                  rows: np.ndarray | None = None) -> np.ndarray:
    """One decoder layer over a micro-batch of tokens at ``start .. start+n-1``.

    Prefill page, ``encode_layer_prefill`` (the whole function):
      1-3c  ``qkv_rows`` for every token,
      3d    K (roped) and V (raw) stored into ``cache[layer][j][start + t]``
            (layer page, ``GpuKvCache``: ``[n_layers][n_kv][max_seq][hd]``),
      3e    causal GQA attention, which sees slots written by earlier tokens of
            this micro-batch and by earlier calls,
      4     ``x += W_o . attn``          (residual GEMM),
      5     FFN RMSNorm,
      6     ``a = silu(gate) * up`` with gate rows ``[0, I)`` and up rows
            ``[I, 2I)`` of the fused weight (layer page: fused = gate ++ up),
      7     ``x += W_down . a``          (residual GEMM).

    ``x`` is ``[n, H]`` float64 and is not modified; the caches are float64
    ``[L][nkv][max_seq][hd]`` and are written in place at exactly the slots
    ``[start, start + n)`` of ``layer``.  Steps 4-7 and the attention are
    per token, so ``rows`` (indices into the micro-batch) limits them to a
    sample; the result is then ``[len(rows), H]``.
    """
    n = x.shape[0]
    positions = start + np.arange(n)
    q, k, v = qkv_rows(shape, w, x, positions)
    k_cache[layer][:, start:start + n, :] = cache_store(shape, k.transpose(1, 0, 2))
    v_cache[layer][:, start:start + n, :] = cache_store(shape, v.transpose(1, 0, 2))
    if rows is None:
        rows = np.arange(n)
    attn = causal_gqa_attention(q[rows], k_cache[layer], v_cache[layer], positions[rows])
    x1 = x[rows] + attn.reshape(len(rows), shape.nq * shape.head_dim) @ as_dense(w["w_o"]).T
    xn2 = rms_norm(x1, w["ffn_norm"], shape.eps)
    gu = xn2 @ as_dense(w["w_gate_up"]).T
    inter = shape.inter
    act = silu(gu[:, :inter]) * gu[:, inter:]
    return x1 + act @ as_dense(w["w_down"]).T


def lm_head_logits(x_last: np.ndarray, final_gain: np.ndarray, eps: float,
                   head: np.ndarray) -> np.ndarray:
    """Logits of the last token: ``W_lm . RMSNorm(x_last; g_final)``.

    Prefill page, ``encode_full_forward_prefill`` "Tail" block (final norm of
    the last token only, then the LM-head GEMV); the chunk page runs the head
    on the last row of the last micro-batch only.
    """
    return as_dense(head) @ rms_norm(x_last, final_gain, eps)


def argmax_rows(logits: np.ndarray) -> np.ndarray:
    """Greedy token per row: the first index of the row's largest logit.

    Prefill page, ``encode_full_forward_prefill``: the greedy branch of the
    tail runs an argmax over the logits on the GPU and hands back one token id.
    The kernel body is not on the pages; ties go to the lowest index (the
    reading taken here), which is what ``numpy.argmax`` returns.
    """
    return np.argmax(np.asarray(logits), axis=-1)


def verify_tail(x_rows: np.ndarray, final_gain: np.ndarray, eps: float, head: np.ndarray):
    """Speculative-verify tail: ``(logits, token ids)`` of every row.

    Prefill page, ``encode_full_forward_prefill_verify``: its tail runs the
    final RMSNorm over all batch positions, the LM-head GEMM on the normed
    rows, then one argmax per position.  Each row is normed on its own.
    """
    logits = rms_norm(np.asarray(x_rows), final_gain, eps) @ as_dense(head).T
    return logits, argmax_rows(logits)


def prefill_chunk(shape, layers: list, x: np.ndarray, start: int, micro_batch: int,
                  k_cache: np.ndarray, v_cache: np.ndarray,
                  final_gain: np.ndarray | None = None, head=None,
                  final_eps: float | None = None):
    """Chunked prefill over every layer: chunk page, ``prefill_chunk_real_llama_dense``.

    The prompt is cut into micro-batches of ``micro_batch`` tokens (the last
    may be shorter); micro-batch ``b`` runs at ``start + offset`` through
    layer 0, 1, ... in order (prefill page, ``encode_full_forward_prefill``
    layer loop), and only after the last micro-batch does the head run on the
    final token.  Returns ``(hidden [n, H], logits or None)``.
    """
    n = x.shape[0]
    mb = micro_batch if micro_batch > 0 else n
    out = np.array(x, dtype=np.float64, copy=True)
    for off in range(0, n, mb):
        xb = out[off:off + mb]
        for layer, w in enumerate(layers):
            xb = prefill_layer(shape, w, layer, xb, start + off, k_cache, v_cache)
        out[off:off + mb] = xb
    logits = None
    if head is not None:
        logits = lm_head_logits(out[-1], final_gain, shape.eps if final_eps is None else final_eps,
                                head)
    return out, logits

