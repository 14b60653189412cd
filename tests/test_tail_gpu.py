"""GPU parity of the token-choice tails: tlp_argmax_rows and tlp_verify_tail.

The argmax decides an integer from floating point, so it is checked where the
decision is unique: bit-exactly against numpy on the same fp32 logits (the
same precision on both sides), and against the float64 oracle's choice
wherever the oracle's top two logits are further apart than twice the
measured logit error.  The verify tail's logits are held to the layer tolerance
(2e-2 bf16, 1e-4 fp32, infinity-norm relative).
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import log, rel_err, tol_of

pytestmark = pytest.mark.gpu


def _tlp():
    import transformer_layer_prefill_amd as tlp
    return tlp


def _argmax_gpu(logits32: np.ndarray, ld: int) -> np.ndarray:
    import torch
    tlp = _tlp()
    rows, vocab = logits32.shape
    buf = np.zeros((rows, ld), dtype=np.float32)
    buf[:, :vocab] = logits32
    d = torch.from_numpy(buf).cuda()
    out = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    tlp.argmax_rows(d, rows, vocab, ld, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_argmax_rows_exact_with_planted_ties():
    rng = np.random.default_rng(11)
    rows, vocab, ld = 37, 1003, 1008
    x = rng.standard_normal((rows, vocab)).astype(np.float32)
    for r in range(0, rows, 3):            # ties: the row maximum at several places
        m = x[r].max() + 1.0
        cols = rng.choice(vocab, size=3, replace=False)
        x[r, cols] = m
    x[5, :] = -np.inf                     # all -inf: index 0
    x[7, :] = 2.0                         # all equal: index 0
    x[8, vocab - 1] = 1e30                # maximum at the last index
    got = _argmax_gpu(x, ld)
    log(f"[parity] argmax rows={rows} vocab={vocab}: {int((got == np.argmax(x, axis=1)).sum())} match")
    np.testing.assert_array_equal(got, np.argmax(x, axis=1))


def test_argmax_rows_never_picks_nan_and_full_vocab():
    rng = np.random.default_rng(12)
    rows, vocab = 3, 128256
    x = rng.standard_normal((rows, vocab)).astype(np.float32)
    x[0, 0] = np.nan
    x[0, 100:200] = np.nan
    x[2, 77] = x[2, 4000] = x[2].max() + 3.0
    got = _argmax_gpu(x, vocab)
    np.testing.assert_array_equal(got, np.nanargmax(x, axis=1))


def _head_shape(name, hidden, vocab, rows, dtype="bf16", seed=2024):
    return synth.Shape(name, hidden=hidden, inter=hidden, nq=1, nkv=1, head_dim=64,
                       qk_norm=False, eps=1e-5, theta=1e4, n_tokens=rows, start=0,
                       max_seq=max(rows, 1), dtype=dtype, vocab=vocab, seed=seed)


def _check_verify(sh):
    import torch
    from transformer_layer_prefill_amd import tensors
    tlp = _tlp()
    x = synth.hidden_input(sh)
    g = synth.final_norm(sh)
    W = synth.lm_head(sh, workers=16)
    cfg = tensors.config_of(sh)
    n, V = sh.n_tokens, sh.vocab
    logits = torch.empty((n, V), dtype=torch.float32, device="cuda")
    tokens = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    ws = torch.empty(tlp.verify_workspace_bytes(cfg, n), dtype=torch.uint8, device="cuda")
    tlp.verify_tail(cfg, tensors.to_device(x), n, tensors.to_device(g), tensors.to_device(W), V,
                    sh.eps, logits, tokens, ws)
    torch.cuda.synchronize()
    g_logits = logits.cpu().numpy()
    g_tokens = tokens.cpu().numpy()
    ref, ref_tokens = oracle.verify_tail(synth.widen(x, sh.dtype), synth.widen(g, sh.dtype),
                                         sh.eps, synth.widen(W, sh.dtype))
    tol = tol_of(sh)
    e = rel_err(g_logits, ref)
    # every GPU logit is within e * max|ref| of the exact one, so where the
    # oracle's top two are more than twice that apart the choice is unique
    srt = np.sort(ref, axis=1)
    bound = 2 * e * np.abs(ref).max()
    sure = (srt[:, -1] - srt[:, -2]) > bound
    log(f"[parity] verify {sh.name}: rows={n} vocab={V} logits={e:.2e} "
        f"decided={int(sure.sum())}/{n}")
    assert e <= tol
    np.testing.assert_array_equal(g_tokens, np.argmax(g_logits, axis=1))
    np.testing.assert_array_equal(g_tokens[sure], ref_tokens[sure])


@pytest.mark.parametrize("rows", [1, 7, 32, 40])
def test_verify_tail_small_bf16(rows):
    # rows <= 32 take the skinny LM-head projection, 40 the tiled GEMM
    _check_verify(_head_shape(f"bf16-h256-v1000-r{rows}", 256, 1000, rows))


def test_verify_tail_small_f32():
    _check_verify(_head_shape("f32-h256-v1003-r5", 256, 1003, 5, dtype="f32"))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("rows", [16, 48])
def test_verify_tail_llama3_head(rows):
    # the Llama-3-8B head: hidden 4096, vocab 128256
    _check_verify(_head_shape(f"llama3-8b-head-r{rows}", 4096, 128256, rows, seed=1004))
