"""Shared plumbing of the GPU parity tests: run the HIP library through the C
ABI on seeded synthetic inputs and run the float64 oracle on the same inputs.

Error metric: for a checked tensor, max|gpu - oracle| / max|oracle| (the
infinity-norm relative error), computed in float64.
"""
from __future__ import annotations

import sys

import numpy as np

import oracle
import synth

BF16_TOL = 2e-2   # bf16 inputs, fp32 accumulation
F32_TOL = 1e-4    # fp32 path


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in the GPU result"
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def tol_of(shape) -> float:
    return F32_TOL if shape.dtype == "f32" else BF16_TOL


class GpuRun:
    """Device-resident inputs of one shape, plus the calls into the library."""

    def __init__(self, shape, layers_np: list, x_np, kc_np, vc_np, device="cuda"):
        import torch
        from transformer_layer_prefill_amd import tensors
        import transformer_layer_prefill_amd as tlp
        self.torch, self.tensors, self.tlp = torch, tensors, tlp
        self.shape = shape
        self.cfg = tensors.config_of(shape)
        self.layers = [tensors.DeviceLayer(w, device) for w in layers_np]
        self.hidden = tensors.to_device(x_np, device)
        self.kc = tensors.to_device(kc_np, device)
        self.vc = tensors.to_device(vc_np, device)
        cos, sin = tlp.rope_table(shape.theta, shape.head_dim, shape.max_seq)
        self.cos = tensors.to_device(cos, device)
        self.sin = tensors.to_device(sin, device)
        self.ws = None

    def pipeline(self):
        """The tlp_pipeline of this run (second stream and events), made once."""
        if getattr(self, "_pipeline", None) is None:
            self._pipeline = self.tlp.Pipeline(self.shape.n_layers)
        return self._pipeline

    def workspace(self, max_tokens, copies=1):
        nbytes = copies * self.tlp.workspace_bytes(self.cfg, max_tokens)
        if self.ws is None or self.ws.numel() < nbytes:
            self.ws = self.torch.empty(nbytes, dtype=self.torch.uint8, device=self.hidden.device)
        return self.ws

    def layer(self, layer: int, n: int, start: int, hidden=None):
        h = self.hidden if hidden is None else hidden
        ws = self.workspace(n)
        self.tlp.prefill_layer(self.cfg, self.layers[layer].struct, layer, h, n, start, self.kc,
                               self.vc, self.cos, self.sin, ws)
        self.torch.cuda.synchronize()

    def chunk(self, n: int, start: int, mb: int, hidden=None, head=None, pipelined=False):
        """pipelined: pass two workspaces' worth of bytes and a pipeline, so
        consecutive micro-batches alternate halves and run on two streams."""
        h = self.hidden if hidden is None else hidden
        copies = 2 if pipelined else 1
        ws = self.workspace(min(n, mb), copies)
        kw = dict(workspace_bytes=copies * self.tlp.workspace_bytes(self.cfg, min(n, mb)))
        if pipelined:
            kw["pipeline"] = self.pipeline()
        if head is not None:
            fn, W, vocab, logits = head
            kw.update(final_norm=fn, lm_head=W, vocab=vocab, final_eps=self.shape.eps,
                      logits=logits)
        self.tlp.prefill_chunk(self.cfg, [d.struct for d in self.layers], h, n, start, mb,
                               self.kc, self.vc, self.cos, self.sin, ws, **kw)
        self.torch.cuda.synchronize()

    def host(self, t):
        return self.tensors.to_host(t)

    def residual_rows(self, n, half=0):
        """fp32 residual stream [n][H] left in the workspace by the last call
        (half 1: the second workspace of a pipelined chunk)."""
        off = half * self.tlp.workspace_bytes(self.cfg, n) + \
            self.tlp.workspace_layout(self.cfg, n)[self.tlp.WS_RES]
        H = self.shape.hidden
        raw = self.ws[off:off + n * H * 4]
        return raw.view(self.torch.float32).reshape(n, H).cpu().numpy().astype(np.float64)


def assert_act_is_rounded_stream(shape, act_rows, res_rows):
    """The hidden rows a call returns are its fp32 residual stream rounded
    once to the activation type: bitwise equal for fp32, and for bf16 the
    round-to-nearest-even of each fp32 value (finite values only)."""
    res = np.ascontiguousarray(res_rows, dtype=np.float32)
    if shape.dtype == "f32":
        assert np.array_equal(np.asarray(act_rows, dtype=np.float32).view(np.uint32),
                              res.view(np.uint32))
        return
    u = res.view(np.uint32).astype(np.uint64)
    rne = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    got = np.asarray(act_rows).view(np.uint16)
    bad = np.flatnonzero(got.ravel() != rne.ravel())
    assert bad.size == 0, (f"{bad.size} hidden values are not the RNE bf16 of the fp32 stream; "
                           f"first at flat index {bad[0]}")


def widen_caches(shape, kc, vc):
    return synth.widen(kc, shape.kv_dtype), synth.widen(vc, shape.kv_dtype)


def oracle_layer(shape, w_np, layer, x_np, kc_np, vc_np, rows=None):
    """Oracle of one layer on storage-format inputs; returns (out, kc64, vc64)."""
    w64 = synth.widen_layer(shape, w_np)
    x64 = synth.widen(x_np, shape.dtype)
    kc64, vc64 = widen_caches(shape, kc_np, vc_np)
    out = oracle.prefill_layer(shape, w64, layer, x64, shape.start, kc64, vc64, rows=rows)
    return out, kc64, vc64


def check_cache_slots(shape, layer, n, start, kc_in, kc_gpu):
    """Bit-exact slot indexing: exactly the slots [start, start+n) of `layer` differ.

    The input caches hold a NaN sentinel in every slot at or after `start`,
    so every written slot must change (to finite values) and every other slot
    must keep its bits.
    """
    u = np.uint32 if kc_in.dtype == np.float32 else np.uint16
    slot_changed = (kc_gpu.view(u) != kc_in.view(u)).any(axis=-1)      # [L][nkv][max_seq]
    expect = np.zeros_like(slot_changed)
    expect[layer, :, start:start + n] = True
    written = synth.widen(kc_gpu[layer, :, start:start + n], shape.kv_dtype)
    assert np.all(np.isfinite(written)), "a written cache slot holds non-finite values"
    assert np.array_equal(slot_changed, expect), "cache slots changed outside [start, start+n)"


def split_kv_boundary_in_window(M, start, nq, nkv):
    """Whether a split-KV key range of the attention launch begins inside the
    query window of one wavefront, with a real query row before the boundary.

    A host-side model of the library's attention launch plan (blocks of one kv
    head and up to four query heads; four or eight wavefronts of 32 query
    rows; key ranges of whole 64-key blocks, about 512 blocks in all when the
    grid alone leaves CUs idle and the cache is at least twice the batch).
    Used only to choose parity cases that cover lanes of one wavefront on both
    sides of a range boundary; the tests never take expected values from it.
    """
    group = nq // nkv
    hpb = min(group, 4)
    quads = group // hpb
    tiles8 = -(-M // (32 * (8 // hpb)))
    waves = 8 if tiles8 * nkv * quads >= 256 else 4
    bt = 32 * (waves // hpb)
    tiles = -(-M // bt)
    blocks = tiles * nkv * quads
    kv_len = start + M
    if waves != 4 or blocks >= 256 or kv_len < 2 * M:
        return False
    nkb = -(-kv_len // 64)
    # the two-key-group form takes over while the keys are few and its grid
    # (twice the blocks) fills the GPU
    if hpb % 2 == 0 and 192 <= 2 * blocks <= 256 and nkb <= 32:
        return False
    ns = min(-(-512 // blocks), 64, nkb // 4)
    if ns < 2:
        return False
    for tile in range(tiles):
        kv_end = start + min(M, (tile + 1) * bt)
        nkb_t = -(-kv_end // 64)
        per = -(-nkb_t // ns)
        for s in range(ns):
            lo = s * per
            if lo >= min(nkb_t, lo + per):
                continue
            for sl in range(waves // hpb):
                t0 = tile * bt + sl * 32
                if any(start + t < lo * 64 for t in range(t0, min(t0 + 32, M))) and \
                        start + t0 + 31 >= lo * 64:
                    return True
    return False
