"""Seeded synthetic inputs for the transformer-layer prefill path.

This module is shared by the tests, ``__graft_entry__.smoke()`` and
``bench.py``.  It draws weights, hidden states and pre-filled KV-cache
contents from seeded generators and rounds them to their storage formats
(fp32, bf16 bit patterns, packed 1-bit signs with fp16 group scales).  It
holds none of the layer's arithmetic: the CPU oracle and the HIP library
each receive the same arrays from here and compute on their own.

Workloads (shapes, value distributions and structure) follow the five
configurations the prefill pages are measured on: a tiny fp32 layer with
QK-norm, a Llama-3-8B-shape bf16 layer, a Qwen3-8B-shape layer with 1-bit
sign weights, a 32-layer 8B-shape stack with a 128256-entry LM head, and a
long-context layer (2048 tokens at position 30720).

Seeds.  Workload ``k`` (1..5) uses base seed ``1000 + k``.  Layer ``l`` of a
workload draws from ``PCG64(base * 1000 + l)`` in the order
attn_norm, w_qkv, q_norm, k_norm, w_o, ffn_norm, w_gate, w_up, w_down, so any
layer can be regenerated alone.  The hidden input, the pre-filled K and V,
the final norm gain and the LM head each have their own stream
``PCG64(base * 1000 + 900 + i)`` for i = 0, 1, 2, 3.

Storage formats.  bf16 arrays are ``numpy.uint16`` bit patterns, rounded
round-to-nearest-even straight from float64.  1-bit weights are a pair
(``bits`` uint32 ``[N][K/32]``, ``scales`` float16 ``[N][K/128]``): bit ``b``
of word ``w`` is the sign of column ``32*w + b`` (1 means +1, 0 means -1) and
each scale covers 128 consecutive columns of one row.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SIGN1_GROUP = 128

# fp32 / bf16 / fp16 NaN patterns that mark cache slots no call has written.
SENTINEL_F32 = np.uint32(0x7FC0DEAD)
SENTINEL_BF16 = np.uint16(0x7FDE)
SENTINEL_F16 = np.uint16(0x7E5A)


@dataclasses.dataclass(frozen=True)
class Shape:
    """One decoder-layer shape plus the prefill call it is exercised with."""

    name: str
    hidden: int
    inter: int
    nq: int
    nkv: int
    head_dim: int
    qk_norm: bool
    eps: float
    theta: float
    n_tokens: int
    start: int
    max_seq: int
    n_layers: int = 1
    dtype: str = "bf16"          # activations, norm gains, KV cache: "f32" | "bf16"
    wformat: str = "dense"       # projection weights: "dense" | "sign1"
    micro_batch: int = 0         # 0: one micro-batch holds every token
    vocab: int = 0               # 0: no LM head
    seed: int = 1000
    kv: str = "act"              # KV-cache format: "act" (= dtype) | "f16"

    @property
    def qkv_dim(self) -> int:
        return (self.nq + 2 * self.nkv) * self.head_dim

    @property
    def q_dim(self) -> int:
        return self.nq * self.head_dim

    @property
    def kv_dtype(self) -> str:
        """Storage type of the KV caches."""
        return "f16" if self.kv == "f16" else self.dtype

    def replace(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


# The five measured workloads.  eps for the 8B shapes is not stated with the
# configurations; 1e-5 (Llama-3) and 1e-6 (Qwen3) are the readings used.
WORKLOADS = {
    "tiny-f32": Shape("tiny-f32", hidden=256, inter=688, nq=4, nkv=2, head_dim=64,
                      qk_norm=True, eps=1e-6, theta=1e4, n_tokens=16, start=0,
                      max_seq=64, dtype="f32", seed=1001),
    "llama3-8b-layer": Shape("llama3-8b-layer", hidden=4096, inter=14336, nq=32, nkv=8,
                             head_dim=128, qk_norm=False, eps=1e-5, theta=5e5,
                             n_tokens=512, start=0, max_seq=4096, seed=1002),
    "qwen3-8b-sign1-layer": Shape("qwen3-8b-sign1-layer", hidden=4096, inter=12288, nq=32,
                                  nkv=8, head_dim=128, qk_norm=True, eps=1e-6, theta=1e6,
                                  n_tokens=512, start=0, max_seq=4096, wformat="sign1",
                                  seed=1003),
    "llama3-8b-stack32": Shape("llama3-8b-stack32", hidden=4096, inter=14336, nq=32, nkv=8,
                               head_dim=128, qk_norm=False, eps=1e-5, theta=5e5,
                               n_tokens=4096, start=0, max_seq=4096, n_layers=32,
                               micro_batch=512, vocab=128256, seed=1004),
    "llama3-8b-long-ctx": Shape("llama3-8b-long-ctx", hidden=4096, inter=14336, nq=32,
                                nkv=8, head_dim=128, qk_norm=False, eps=1e-5, theta=5e5,
                                n_tokens=2048, start=30720, max_seq=32768, seed=1005),
    # token-by-token decode steps of the same layer: one token after a full
    # 4096-slot context, and after a 32767-slot context
    "llama3-8b-decode": Shape("llama3-8b-decode", hidden=4096, inter=14336, nq=32, nkv=8,
                              head_dim=128, qk_norm=False, eps=1e-5, theta=5e5,
                              n_tokens=1, start=4095, max_seq=4096, seed=1002),
    "llama3-8b-long-decode": Shape("llama3-8b-long-decode", hidden=4096, inter=14336, nq=32,
                                   nkv=8, head_dim=128, qk_norm=False, eps=1e-5, theta=5e5,
                                   n_tokens=1, start=32767, max_seq=32768, seed=1005),
}


# ---------------------------------------------------------------------------
# storage-format rounding (input preparation only)
# ---------------------------------------------------------------------------

def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even) and return the bits.

    Works on the float64 bit pattern directly so no intermediate float32
    rounding can double-round.  Inputs must be finite and inside the bf16
    normal range (true for every distribution drawn here).
    """
    b = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)
    lsb = (b >> np.uint64(45)) & np.uint64(1)
    b = (b + np.uint64(0xFFFFFFFFFFF) + lsb) & ~np.uint64((1 << 45) - 1)
    f32 = b.view(np.float64).astype(np.float32)        # exact: 8 significant bits
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float64 exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x64.astype(np.float32)
    if dtype == "bf16":
        return f64_to_bf16_bits(x64)
    if dtype == "f16":
        return x64.astype(np.float16)      # nearest-even
    raise ValueError(dtype)


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored activation/gain array -> exact float64."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    if dtype == "f16":
        return np.asarray(a, dtype=np.float16).astype(np.float64)
    raise ValueError(dtype)


def sentinel(dtype: str):
    if dtype == "f16":
        return SENTINEL_F16.view(np.float16)
    return SENTINEL_F32 if dtype == "f32" else SENTINEL_BF16


def storage_np_dtype(dtype: str):
    return {"f32": np.float32, "bf16": np.uint16, "f16": np.float16}[dtype]


# ---------------------------------------------------------------------------
# draws
# ---------------------------------------------------------------------------

def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _gain(rng, n, dtype):
    return to_storage(1.0 + 0.05 * rng.standard_normal(n), dtype)


def _dense(rng, n, k, dtype):
    return to_storage(0.02 * rng.standard_normal((n, k)), dtype)


def _sign1(rng, n, k):
    if k % SIGN1_GROUP:
        raise ValueError(f"1-bit weights need K % {SIGN1_GROUP} == 0, got K={k}")
    bits = rng.integers(0, 1 << 32, size=(n, k // 32), dtype=np.uint32)
    scales = np.abs(0.02 * rng.standard_normal((n, k // SIGN1_GROUP))).astype(np.float16)
    return {"bits": bits, "scales": scales}


def layer_weights(shape: Shape, layer: int) -> dict:
    """Weights of one layer in storage format.

    Keys: attn_norm [H], w_qkv [(nq+2nkv)hd x H], q_norm [hd], k_norm [hd],
    w_o [H x nq*hd], ffn_norm [H], w_gate_up [2I x H] (gate rows first),
    w_down [H x I].  With ``wformat == "sign1"`` each projection is a
    ``{"bits", "scales"}`` dict instead of a dense array.
    """
    rng = _rng(shape.seed * 1000 + layer)
    H, I, hd, dt = shape.hidden, shape.inter, shape.head_dim, shape.dtype
    proj = (lambda n, k: _sign1(rng, n, k)) if shape.wformat == "sign1" else \
        (lambda n, k: _dense(rng, n, k, dt))
    w = {}
    w["attn_norm"] = _gain(rng, H, dt)
    w["w_qkv"] = proj(shape.qkv_dim, H)
    w["q_norm"] = _gain(rng, hd, dt)
    w["k_norm"] = _gain(rng, hd, dt)
    w["w_o"] = proj(H, shape.q_dim)
    w["ffn_norm"] = _gain(rng, H, dt)
    gate = proj(I, H)
    up = proj(I, H)
    if shape.wformat == "sign1":
        w["w_gate_up"] = {k: np.concatenate([gate[k], up[k]], axis=0) for k in gate}
    else:
        w["w_gate_up"] = np.concatenate([gate, up], axis=0)
    del gate, up
    w["w_down"] = proj(H, I)
    return w


def stack_weights(shape: Shape, workers: int = 8) -> list:
    """All layers' weights, drawn in parallel (each layer has its own stream)."""
    with ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        return list(ex.map(lambda l: layer_weights(shape, l), range(shape.n_layers)))


def hidden_input(shape: Shape, n_tokens: int | None = None) -> np.ndarray:
    n = shape.n_tokens if n_tokens is None else n_tokens
    rng = _rng(shape.seed * 1000 + 900)
    return to_storage(rng.standard_normal((n, shape.hidden)), shape.dtype)


def kv_caches(shape: Shape) -> tuple[np.ndarray, np.ndarray]:
    """K and V caches ``[L][nkv][max_seq][hd]`` in storage format.

    Slots below ``shape.start`` hold N(0,1) values (an earlier prompt's keys
    and values); every other slot holds a NaN sentinel, so reading a slot no
    call has written poisons the result.
    """
    L, nkv, S, hd, s = shape.n_layers, shape.nkv, shape.max_seq, shape.head_dim, shape.start
    rng = _rng(shape.seed * 1000 + 901)
    kd = shape.kv_dtype
    out = []
    for _ in range(2):
        c = np.full((L, nkv, S, hd), sentinel(kd), dtype=storage_np_dtype(kd))
        if s:
            vals = rng.standard_normal((L, nkv, s, hd))
            c[:, :, :s, :] = to_storage(vals, kd).view(c.dtype)
        out.append(c)
    return out[0], out[1]


def final_norm(shape: Shape) -> np.ndarray:
    return _gain(_rng(shape.seed * 1000 + 902), shape.hidden, shape.dtype)


def lm_head(shape: Shape, workers: int = 8) -> np.ndarray:
    """``[vocab x H]`` ~ N(0, 0.02), drawn in row blocks with one stream per block."""
    V, H = shape.vocab, shape.hidden
    block = 8192
    starts = list(range(0, V, block))

    def draw(i):
        r0 = starts[i]
        rng = _rng((shape.seed * 1000 + 903) * 1000 + i)
        return _dense(rng, min(block, V - r0), H, shape.dtype)

    with ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        parts = list(ex.map(draw, range(len(starts))))
    return np.concatenate(parts, axis=0)


# ---------------------------------------------------------------------------
# float64 views for the oracle
# ---------------------------------------------------------------------------

def sign1_to_f64_parts(wq: dict) -> tuple[np.ndarray, np.ndarray]:
    """(bits uint32, scales float64) of a 1-bit weight; decoding is the oracle's job."""
    return wq["bits"], wq["scales"].astype(np.float64)


def widen_layer(shape: Shape, w: dict) -> dict:
    """Storage-format layer weights -> float64 arrays (dense) or (bits, scales64)."""
    out = {}
    for k, v in w.items():
        if isinstance(v, dict):
            out[k] = sign1_to_f64_parts(v)
        else:
            out[k] = widen(v, shape.dtype)
    return out
