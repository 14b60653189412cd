"""The workspace-free layer entry point (tlp_prefill_layer_noalloc) against
the workspace one, through the C ABI: two calls in a row, the second smaller
and continuing the first's cache, each bit-identical to tlp_prefill_layer on
the same inputs and within 2e-2 of the float64 oracle."""
import numpy as np
import pytest

import oracle
import synth
from helpers import GpuRun, check_cache_slots, log, rel_err, widen_caches

pytestmark = pytest.mark.gpu


def _shape():
    return synth.Shape("noalloc", hidden=512, inter=1024, nq=8, nkv=2, head_dim=128,
                       qk_norm=True, eps=1e-6, theta=1e6, n_tokens=96, start=40, max_seq=160,
                       seed=31)


def test_noalloc_matches_workspace_entry_point():
    import torch
    sh = _shape()
    w = synth.layer_weights(sh, 0)
    calls = [(96, 40), (20, 136)]     # the second continues the first, fewer tokens
    x_all = synth.hidden_input(sh, 116)
    kc, vc = synth.kv_caches(sh)
    ref = GpuRun(sh, [w], x_all[:96], kc, vc)      # workspace entry point
    got = GpuRun(sh, [w], x_all[:96], kc, vc)      # static scratch entry point
    w64 = synth.widen_layer(sh, w)
    kc64, vc64 = widen_caches(sh, kc, vc)
    off = 0
    for n, start in calls:
        log(f"[noalloc] call n={n} start={start}")
        x = x_all[off:off + n]
        from transformer_layer_prefill_amd import tensors
        h_ref = tensors.to_device(x)
        h_got = tensors.to_device(x)
        ref.layer(0, n, start, hidden=h_ref)
        got.tlp.prefill_layer_noalloc(got.cfg, got.layers[0].struct, 0, h_got, n, start,
                                      got.kc, got.vc, got.cos, got.sin)
        torch.cuda.synchronize()
        a, b = got.host(h_got), ref.host(h_ref)
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), "hidden differs"
        for c_got, c_ref in ((got.kc, ref.kc), (got.vc, ref.vc)):
            assert np.array_equal(got.host(c_got).view(np.uint16), ref.host(c_ref).view(np.uint16))
        out = oracle.prefill_layer(sh, w64, 0, synth.widen(x, sh.dtype), start, kc64, vc64)
        e = rel_err(synth.widen(a, sh.dtype), out)
        e_k = rel_err(synth.widen(got.host(got.kc)[0, :, start:start + n], sh.kv_dtype),
                      kc64[0, :, start:start + n])
        log(f"[noalloc] n={n}: hidden={e:.2e} k={e_k:.2e}")
        assert e <= 2e-2 and e_k <= 2e-2
        off += n
    # exactly the slots of the two calls were written
    for c_in, c_gpu in ((kc, got.host(got.kc)), (vc, got.host(got.vc))):
        check_cache_slots(sh, 0, 116, 40, c_in, c_gpu)


def test_noalloc_rejects_oversize_call_on_gpu():
    import transformer_layer_prefill_amd as tlp
    sh = synth.WORKLOADS["llama3-8b-layer"]
    w = synth.layer_weights(sh.replace(n_tokens=1), 0)
    x = synth.hidden_input(sh, 512)
    kc, vc = synth.kv_caches(sh.replace(max_seq=512))
    gpu = GpuRun(sh.replace(max_seq=512), [w], x, kc, vc)
    with pytest.raises(tlp.TlpError) as err:
        gpu.tlp.prefill_layer_noalloc(gpu.cfg, gpu.layers[0].struct, 0, gpu.hidden, 512, 0,
                                      gpu.kc, gpu.vc, gpu.cos, gpu.sin)
    assert err.value.status == tlp.TLP_ERR_WORKSPACE
