"""C-ABI checks that need no GPU: the library loads, exports every function
include/tlp.h declares, rejects invalid arguments before enqueuing anything,
and its host-side RoPE table matches the closed form.

Every prefill call here fails validation, so no kernel is ever launched
(the device pointers are fake, aligned, non-null addresses).
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import synth
import transformer_layer_prefill_amd as tlp
from transformer_layer_prefill_amd import tensors

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tlp.h")
FAKE = 1 << 20          # 256-aligned, non-null, never dereferenced


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tlp_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    declared = _declared_functions()
    assert set(declared) == set(tlp.EXPORTS)
    L = tlp.lib()
    for name in declared:
        assert hasattr(L, name), name


def _cfg(**kw):
    base = dict(hidden=256, intermediate=688, n_q_heads=4, n_kv_heads=2, head_dim=64,
                max_seq=64, n_layers=2, rms_eps=1e-6, qk_norm=1, dtype=tlp.TLP_BF16,
                wformat=tlp.TLP_W_DENSE)
    base.update(kw)
    return tlp.make_config(**base)


def _weights(null=None):
    w = tlp.LayerWeights()
    for k in ("attn_norm", "q_norm", "k_norm", "ffn_norm"):
        setattr(w, k, None if k == null else FAKE)
    for k in ("w_qkv", "w_o", "w_gate_up", "w_down"):
        setattr(w, k, tlp.Weight(None if k == null else FAKE, FAKE))
    return w


def _layer(cfg, w=None, layer=0, n=4, start=0, ws_bytes=None, hidden=FAKE, ws=FAKE, kc=FAKE,
           rope=FAKE):
    w = w if w is not None else _weights()
    wsb = tlp.workspace_bytes(cfg, max(n, 1)) if ws_bytes is None else ws_bytes
    L = tlp.lib()
    st = L.tlp_prefill_layer(ctypes.byref(cfg), ctypes.byref(w), layer, hidden, n, start, kc,
                             FAKE, rope, FAKE, ws, wsb, None)
    return st, L.tlp_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), tlp.TLP_ERR_SHAPE),
    (dict(n_q_heads=6, n_kv_heads=4), tlp.TLP_ERR_SHAPE),
    (dict(n_q_heads=6, n_kv_heads=2), tlp.TLP_ERR_UNSUPPORTED),
    (dict(hidden=260), tlp.TLP_ERR_SHAPE),
    (dict(intermediate=690), tlp.TLP_ERR_SHAPE),
    (dict(dtype=7), tlp.TLP_ERR_UNSUPPORTED),
    (dict(wformat=tlp.TLP_W_SIGN1_G128, dtype=tlp.TLP_F32), tlp.TLP_ERR_UNSUPPORTED),
    (dict(wformat=tlp.TLP_W_SIGN1_G128), tlp.TLP_ERR_SHAPE),   # I = 688 is not % 128
    (dict(rms_eps=float("nan")), tlp.TLP_ERR_SHAPE),
    (dict(max_seq=0), tlp.TLP_ERR_SHAPE),
])
def test_invalid_config_rejected(kw, status):
    st, msg = _layer(_cfg(**kw), ws_bytes=1 << 30)
    assert st == status, msg
    assert msg


def test_call_argument_checks():
    cfg = _cfg()
    assert _layer(cfg, n=0)[0] == tlp.TLP_ERR_SHAPE                 # empty chunk
    assert _layer(cfg, start=-1)[0] == tlp.TLP_ERR_POSITION
    assert _layer(cfg, start=61, n=4)[0] == tlp.TLP_ERR_POSITION     # 61 + 4 > 64
    assert _layer(cfg, layer=2)[0] == tlp.TLP_ERR_SHAPE
    assert _layer(cfg, layer=-1)[0] == tlp.TLP_ERR_SHAPE
    assert _layer(cfg, hidden=None)[0] == tlp.TLP_ERR_NULL
    assert _layer(cfg, hidden=FAKE + 8)[0] == tlp.TLP_ERR_UNSUPPORTED   # misaligned
    assert _layer(cfg, ws=FAKE + 16)[0] == tlp.TLP_ERR_WORKSPACE
    need = tlp.workspace_bytes(cfg, 4)
    st, msg = _layer(cfg, ws_bytes=need - 1)
    assert st == tlp.TLP_ERR_WORKSPACE and str(need) in msg
    for k in ("attn_norm", "ffn_norm", "w_qkv", "w_o", "w_gate_up", "w_down", "q_norm"):
        assert _layer(cfg, w=_weights(null=k))[0] == tlp.TLP_ERR_NULL, k
    # the RoPE/KV kernel reads gains and rope tables with vector loads
    assert _layer(cfg, rope=FAKE + 4)[0] == tlp.TLP_ERR_UNSUPPORTED
    w = _weights()
    w.q_norm = FAKE + 8
    assert _layer(cfg, w=w)[0] == tlp.TLP_ERR_UNSUPPORTED
    # q_norm may be NULL when QK-norm is off
    cfg_off = _cfg(qk_norm=0)
    assert _layer(cfg_off, w=_weights(null="q_norm"), n=0)[0] == tlp.TLP_ERR_SHAPE


def test_sign1_needs_scales():
    cfg = _cfg(wformat=tlp.TLP_W_SIGN1_G128, hidden=256, intermediate=512)
    w = _weights()
    w.w_o = tlp.Weight(FAKE, None)
    assert _layer(cfg, w=w)[0] == tlp.TLP_ERR_NULL


def test_chunk_argument_checks():
    cfg = _cfg()
    L = tlp.lib()
    arr = (tlp.LayerWeights * 2)(_weights(), _weights())
    wsb = tlp.workspace_bytes(cfg, 4)

    def chunk(n=8, mb=4, head=None, norm=FAKE, logits=FAKE, vocab=10, layers=arr, wsb=wsb):
        return L.tlp_prefill_chunk(ctypes.byref(cfg), layers, FAKE, n, 0, mb, FAKE, FAKE, FAKE,
                                   FAKE, norm, head, vocab, 1e-5, logits, FAKE, wsb, None, None)

    assert chunk(mb=0) == tlp.TLP_ERR_SHAPE
    assert chunk(head=FAKE, norm=None) == tlp.TLP_ERR_NULL
    assert chunk(head=FAKE, logits=None) == tlp.TLP_ERR_NULL
    assert chunk(head=FAKE, vocab=0) == tlp.TLP_ERR_SHAPE
    assert chunk(wsb=wsb - 256) == tlp.TLP_ERR_WORKSPACE
    assert chunk(layers=None) == tlp.TLP_ERR_NULL
    bad = (tlp.LayerWeights * 2)(_weights(), _weights(null="w_down"))
    assert chunk(layers=bad) == tlp.TLP_ERR_NULL


def test_argmax_and_verify_argument_checks():
    L = tlp.lib()
    assert L.tlp_argmax_rows(None, 2, 10, 10, FAKE, None) == tlp.TLP_ERR_NULL
    assert L.tlp_argmax_rows(FAKE, 2, 10, 10, None, None) == tlp.TLP_ERR_NULL
    assert L.tlp_argmax_rows(FAKE, 0, 10, 10, FAKE, None) == tlp.TLP_ERR_SHAPE
    assert L.tlp_argmax_rows(FAKE, 2, 0, 10, FAKE, None) == tlp.TLP_ERR_SHAPE
    assert L.tlp_argmax_rows(FAKE, 2, 10, 9, FAKE, None) == tlp.TLP_ERR_SHAPE
    cfg = _cfg()
    assert tlp.verify_workspace_bytes(cfg, 0) == 0
    assert tlp.verify_workspace_bytes(cfg, 3) == 1536   # bf16 [3][256], 256-byte multiple
    wsb = tlp.verify_workspace_bytes(cfg, 3)

    def verify(n=3, norm=FAKE, head=FAKE, vocab=10, logits=FAKE, ws=FAKE, wsb=wsb, eps=1e-5):
        return L.tlp_verify_tail(ctypes.byref(cfg), FAKE, n, norm, head, vocab, eps, logits,
                                 None, ws, wsb, None)

    assert verify(head=None) == tlp.TLP_ERR_NULL
    assert verify(norm=None) == tlp.TLP_ERR_NULL
    assert verify(logits=None) == tlp.TLP_ERR_NULL
    assert verify(n=0) == tlp.TLP_ERR_SHAPE
    assert verify(vocab=0) == tlp.TLP_ERR_SHAPE
    assert verify(eps=-1.0) == tlp.TLP_ERR_SHAPE
    assert verify(logits=FAKE + 4) == tlp.TLP_ERR_UNSUPPORTED
    assert verify(ws=FAKE + 16) == tlp.TLP_ERR_UNSUPPORTED
    assert verify(wsb=wsb - 1) == tlp.TLP_ERR_WORKSPACE


def test_workspace_sizes():
    cfg = _cfg()
    assert tlp.workspace_bytes(cfg, 0) == 0
    offs = tlp.workspace_layout(cfg, 16)
    assert offs[0] == 0 and all(b > a for a, b in zip(offs, offs[1:]))
    assert all(o % 256 == 0 for o in offs)
    # RES is fp32 [16][256]; XN bf16 [16][256]; QKV bf16 [16][(4+4)*64]
    assert offs[tlp.WS_XN] == 16 * 256 * 4
    assert offs[tlp.WS_QKV] - offs[tlp.WS_XN] == 16 * 256 * 2
    assert tlp.workspace_bytes(cfg, 16) >= offs[-1] + 256 * 4
    assert tlp.workspace_bytes(cfg, 32) > tlp.workspace_bytes(cfg, 16)


def test_status_strings():
    L = tlp.lib()
    for s in range(7):
        assert L.tlp_status_string(s)


def test_rope_table_closed_form():
    theta, hd, n = 5e5, 128, 40000
    cos, sin = tlp.rope_table(theta, hd, n)
    assert cos.shape == (n, 64)
    # position 0: cos 1, sin 0 exactly
    assert np.all(cos[0] == 1.0) and np.all(sin[0] == 0.0)
    # frequency 0 is exactly 1 rad per position; pair i has theta^(-2i/hd)
    for p, i in [(1, 0), (7, 0), (31000, 0), (12345, 17), (32767, 63)]:
        ang = p * theta ** (-2.0 * i / hd)
        assert cos[p, i] == np.float32(math.cos(ang))
        assert sin[p, i] == np.float32(math.sin(ang))
    np.testing.assert_allclose(cos.astype(np.float64) ** 2 + sin.astype(np.float64) ** 2, 1.0,
                               atol=2e-7)


def test_rope_table_rejects_bad_args():
    with pytest.raises(tlp.TlpError):
        tlp.rope_table(1e4, 63, 10)
    with pytest.raises(tlp.TlpError):
        tlp.rope_table(-1.0, 64, 10)


def test_config_of_workloads():
    for shape in synth.WORKLOADS.values():
        cfg = tensors.config_of(shape)
        assert tlp.workspace_bytes(cfg, shape.micro_batch or shape.n_tokens) > 0


def test_stored_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    """bench.stored_traffic reports committed counters only while the source
    files named by the counter entry hash as they did when it was taken."""
    import json
    import bench
    now = {"gemm.hip": "a", "skinny.hip": "b", "common.h": "c"}
    entry = {"fetch_bytes": 10.0, "write_bytes": 2.0, "sources": ["skinny.hip", "common.h"]}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic_w.json").write_text(json.dumps(
        {"source_sha256": now, "kernels": {"gate_up_gemm | sym": entry}}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_sha256", lambda: dict(now))
    assert bench.stored_traffic("w", "gate_up_gemm")["bytes"] == 12
    assert bench.stored_traffic("w", "down_gemm") is None
    assert bench.stored_traffic("missing", "gate_up_gemm") is None
    # a file the entry does not name may change; one it names may not
    monkeypatch.setattr(bench, "source_sha256", lambda: dict(now, **{"gemm.hip": "x"}))
    assert bench.stored_traffic("w", "gate_up_gemm")["bytes"] == 12
    monkeypatch.setattr(bench, "source_sha256", lambda: dict(now, **{"skinny.hip": "x"}))
    assert bench.stored_traffic("w", "gate_up_gemm") is None


def test_bench_refuses_more_than_one_gpu():
    """The bench measures one GPU; asking for more ends with a message, not a run."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_noalloc_rejects_calls_beyond_its_scratch():
    # an 8B-shape layer at 512 tokens needs ~100 MiB of workspace, above the
    # 64 MiB static scratch: rejected before the device is touched
    sh = synth.WORKLOADS["llama3-8b-layer"]
    cfg = tensors.config_of(sh)
    assert tlp.workspace_bytes(cfg, 512) > tlp.NOALLOC_SCRATCH_BYTES
    L = tlp.lib()
    w = _weights()
    st = L.tlp_prefill_layer_noalloc(ctypes.byref(cfg), ctypes.byref(w), 0, FAKE, 512, 0, FAKE,
                                     FAKE, FAKE, FAKE, None)
    msg = L.tlp_last_error().decode()
    assert st == tlp.TLP_ERR_WORKSPACE, msg
    assert str(tlp.NOALLOC_SCRATCH_BYTES) in msg
    # the usual argument checks come first
    assert L.tlp_prefill_layer_noalloc(ctypes.byref(cfg), ctypes.byref(w), 0, FAKE, 0, 0, FAKE,
                                       FAKE, FAKE, FAKE, None) == tlp.TLP_ERR_SHAPE
    assert L.tlp_prefill_layer_noalloc(ctypes.byref(cfg), ctypes.byref(_weights(null="w_o")), 0,
                                       FAKE, 4, 0, FAKE, FAKE, FAKE, FAKE,
                                       None) == tlp.TLP_ERR_NULL


def test_pipeline_and_profiler_argument_checks():
    # rejected before any HIP call: no stream or event is created
    L = tlp.lib()
    h = ctypes.c_void_p(123)
    assert L.tlp_pipeline_create(0, ctypes.byref(h)) == tlp.TLP_ERR_SHAPE
    assert h.value is None                      # *out is cleared on failure
    assert L.tlp_pipeline_create(4, None) == tlp.TLP_ERR_NULL
    assert L.tlp_pipeline_destroy(None) == tlp.TLP_OK
    assert L.tlp_profile_begin(0) == tlp.TLP_ERR_SHAPE
    assert L.tlp_profile_end(None, None, None) == tlp.TLP_ERR_NULL
