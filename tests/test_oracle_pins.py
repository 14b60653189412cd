"""Pins of the CPU float64 oracle to facts outside itself.

Each test checks the oracle against something the pages or the mathematics
fix: hand-worked values (tests/golden/hand_cases.json), closed forms,
invariants, special cases that reduce to something simpler, and brute force
over explicit index loops on tiny inputs.  The shapes are deliberately
non-square (H != nq*hd, I != H) so a transposed weight fails on shape.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")
MATH_NS = {"sqrt": math.sqrt, "cos": math.cos, "sin": math.sin, "exp": math.exp}


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _eval(exprs):
    return np.array([eval(e, {"__builtins__": {}}, MATH_NS) for e in exprs], dtype=np.float64)


# ---------------------------------------------------------------- RMSNorm

@pytest.mark.parametrize("case", _golden()["rmsnorm"])
def test_rmsnorm_hand_cases(case):
    got = oracle.rms_norm(np.array(case["x"]), np.array(case["gain"]), case["eps"])
    np.testing.assert_allclose(got, _eval(case["expected"]), rtol=1e-15, atol=1e-15)


def test_rmsnorm_output_rms_closed_form():
    # unit gain: rms(out) = sqrt(ms / (ms + eps)) for every row
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 33)) * 0.7
    eps = 0.3
    out = oracle.rms_norm(x, np.ones(33), eps)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.sqrt(np.mean(out * out, axis=1)), np.sqrt(ms / (ms + eps)),
                               rtol=1e-14)


def test_rmsnorm_scale_invariant_at_zero_eps():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 40))
    g = 1 + 0.05 * rng.standard_normal(40)
    np.testing.assert_allclose(oracle.rms_norm(7.5 * x, g, 0.0), oracle.rms_norm(x, g, 0.0),
                               rtol=1e-14)


# ---------------------------------------------------------------- RoPE

@pytest.mark.parametrize("case", _golden()["rope"])
def test_rope_hand_cases(case):
    x = np.array(case["x"], dtype=np.float64)[None, None, :]
    got = oracle.apply_rope(x, np.array([case["position"]]), case["theta"])[0, 0]
    np.testing.assert_allclose(got, _eval(case["expected"]), rtol=1e-15, atol=1e-15)


def test_rope_position_zero_is_identity_bitwise():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 5, 64))
    out = oracle.apply_rope(x, np.zeros(3, dtype=np.int64), 5e5)
    assert np.array_equal(out, x)


def test_rope_preserves_pair_and_head_norms():
    rng = np.random.default_rng(3)
    hd = 128
    x = rng.standard_normal((9, 4, hd))
    pos = np.array([0, 1, 7, 100, 511, 4095, 30720, 32767, 12345])
    out = oracle.apply_rope(x, pos, 5e5)
    h = hd // 2
    np.testing.assert_allclose(out[..., :h] ** 2 + out[..., h:] ** 2,
                               x[..., :h] ** 2 + x[..., h:] ** 2, rtol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(out, axis=-1), np.linalg.norm(x, axis=-1),
                               rtol=1e-13)


def test_rope_depends_on_relative_position_only():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))

    def dot(p, pk):
        return float(np.sum(oracle.apply_rope(q, np.array([p]), 1e4) *
                            oracle.apply_rope(k, np.array([pk]), 1e4)))

    for p, pk, d in [(5, 2, 11), (100, 0, 300), (17, 17, 1000)]:
        assert dot(p, pk) == pytest.approx(dot(p + d, pk + d), rel=1e-10, abs=1e-12)


# ---------------------------------------------------------------- SiLU / SwiGLU

def test_silu_hand_cases():
    case = _golden()["silu"][0]
    np.testing.assert_allclose(oracle.silu(np.array(case["z"])), _eval(case["expected"]),
                               rtol=1e-15, atol=0)


def test_silu_limits():
    assert oracle.silu(np.array([40.0]))[0] == pytest.approx(40.0, rel=1e-15)
    assert abs(oracle.silu(np.array([-40.0]))[0]) < 1e-15


# ---------------------------------------------------------------- 1-bit decode

def test_sign1_hand_case():
    case = _golden()["sign1"][0]
    bits = np.array([case["words"]], dtype=np.uint32)
    scales = np.array([[case["scale"]]], dtype=np.float64)
    w = oracle.decode_sign1(bits, scales)[0]
    expect = np.full(128, -case["scale"])
    expect[case["plus_columns"]] = case["scale"]
    assert np.array_equal(w, expect)


def test_sign1_all_ones_gives_scaled_group_sums():
    # every bit set: W[o][k] = s[o][k // 128], so Y[t][o] = sum_g s[o][g] * sum_{k in g} X[t][k]
    rng = np.random.default_rng(5)
    n, k = 6, 384
    bits = np.full((n, k // 32), 0xFFFFFFFF, dtype=np.uint32)
    scales = rng.standard_normal((n, k // 128))   # signed: any fp16 scale is allowed
    x = rng.standard_normal((4, k))
    y = x @ oracle.decode_sign1(bits, scales).T
    group_sums = x.reshape(4, 3, 128).sum(axis=2)          # [t, g]
    np.testing.assert_allclose(y, group_sums @ scales.T, rtol=1e-12)


def test_sign1_negating_all_bits_negates_weights():
    rng = np.random.default_rng(6)
    bits = rng.integers(0, 1 << 32, size=(5, 8), dtype=np.uint32)
    scales = rng.standard_normal((5, 2))
    assert np.array_equal(oracle.decode_sign1(~bits, scales), -oracle.decode_sign1(bits, scales))


# ---------------------------------------------------------------- attention

def _brute_attention(q, kc, vc, positions):
    """Explicit index loops: per query row, head and key."""
    r, nq, hd = q.shape
    nkv = kc.shape[0]
    out = np.zeros((r, nq, hd))
    for i in range(r):
        for h in range(nq):
            j = h * nkv // nq
            s = [sum(q[i, h, d] * kc[j, u, d] for d in range(hd)) / math.sqrt(hd)
                 for u in range(positions[i] + 1)]
            m = max(s)
            e = [math.exp(v - m) for v in s]
            tot = sum(e)
            for d in range(hd):
                out[i, h, d] = sum(e[u] * vc[j, u, d] for u in range(len(e))) / tot
    return out


def test_attention_matches_brute_force():
    rng = np.random.default_rng(7)
    nq, nkv, hd, S = 6, 2, 8, 12
    q = rng.standard_normal((5, nq, hd))
    kc = rng.standard_normal((nkv, S, hd))
    vc = rng.standard_normal((nkv, S, hd))
    pos = np.array([0, 3, 4, 9, 11])
    np.testing.assert_allclose(oracle.causal_gqa_attention(q, kc, vc, pos),
                               _brute_attention(q, kc, vc, pos), rtol=1e-12, atol=1e-13)


def test_attention_first_token_returns_v0():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 4, 16))
    kc = rng.standard_normal((2, 5, 16))
    vc = rng.standard_normal((2, 5, 16))
    out = oracle.causal_gqa_attention(q, kc, vc, np.array([0]))
    assert np.array_equal(out[0, :2], np.broadcast_to(vc[0, 0], (2, 16)))
    assert np.array_equal(out[0, 2:], np.broadcast_to(vc[1, 0], (2, 16)))


def test_attention_equal_keys_gives_mean_of_visible_values():
    rng = np.random.default_rng(9)
    kc = np.broadcast_to(rng.standard_normal(16), (1, 10, 16)).copy()
    vc = rng.standard_normal((1, 10, 16))
    q = rng.standard_normal((3, 2, 16))
    pos = np.array([2, 5, 9])
    out = oracle.causal_gqa_attention(q, kc, vc, pos)
    for i, p in enumerate(pos):
        np.testing.assert_allclose(out[i, 0], vc[0, :p + 1].mean(axis=0), rtol=1e-13)


def test_attention_gqa_head_mapping():
    # kv head j holds the constant value j: query head h must read kv head h // (nq/nkv)
    nq, nkv, hd = 8, 4, 4
    rng = np.random.default_rng(10)
    vc = np.zeros((nkv, 6, hd)) + np.arange(nkv)[:, None, None]
    kc = rng.standard_normal((nkv, 6, hd))
    q = rng.standard_normal((2, nq, hd))
    out = oracle.causal_gqa_attention(q, kc, vc, np.array([3, 5]))
    for h in range(nq):
        np.testing.assert_allclose(out[:, h], h // 2, atol=1e-14)


def test_attention_mha_when_nq_equals_nkv():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((3, 3, 8))
    kc = rng.standard_normal((3, 7, 8))
    vc = rng.standard_normal((3, 7, 8))
    pos = np.array([1, 4, 6])
    out = oracle.causal_gqa_attention(q, kc, vc, pos)
    for h in range(3):
        np.testing.assert_allclose(out[:, h:h + 1],
                                   oracle.causal_gqa_attention(q[:, h:h + 1], kc[h:h + 1],
                                                               vc[h:h + 1], pos)[:, 0:1],
                                   rtol=1e-14)


# ---------------------------------------------------------------- the layer

TINY = synth.Shape("pin", hidden=96, inter=40, nq=4, nkv=2, head_dim=16, qk_norm=True,
                   eps=1e-6, theta=1e4, n_tokens=9, start=0, max_seq=32, n_layers=2,
                   dtype="f32", seed=77)


def _tiny_weights(shape):
    return [synth.widen_layer(shape, synth.layer_weights(shape, l)) for l in range(shape.n_layers)]


def _nan_caches(shape):
    c = np.full((shape.n_layers, shape.nkv, shape.max_seq, shape.head_dim), np.nan)
    return c, c.copy()


def test_layer_zero_output_projections_pass_residual_through():
    ws = _tiny_weights(TINY)[0]
    ws["w_o"] = np.zeros_like(ws["w_o"])
    ws["w_down"] = np.zeros_like(ws["w_down"])
    x = np.random.default_rng(12).standard_normal((5, TINY.hidden))
    kc, vc = _nan_caches(TINY)
    assert np.array_equal(oracle.prefill_layer(TINY, ws, 0, x, 0, kc, vc), x)


def test_layer_writes_exactly_the_slots_of_its_tokens():
    ws = _tiny_weights(TINY)
    kc, vc = _nan_caches(TINY)
    x = np.random.default_rng(13).standard_normal((6, TINY.hidden))
    kc[:, :, :4] = 0.25
    vc[:, :, :4] = -0.5
    oracle.prefill_layer(TINY, ws[1], 1, x, 4, kc, vc)
    written = ~np.isnan(kc)
    expect = np.zeros_like(written)
    expect[:, :, :4] = True
    expect[1, :, 4:10] = True
    assert np.array_equal(written, expect)
    assert np.array_equal(~np.isnan(vc), expect)
    assert np.all(kc[0, :, :4] == 0.25)


def test_layer_k_slot_holds_key_roped_at_its_absolute_position():
    # constant hidden rows, unit gains, eps 0: xn is the all-ones row; W_k row 0 of
    # kv head j is 1/H, every other K row 0, so the pre-RoPE key is e_0 and the
    # roped key at absolute position p is cos(p) on element 0, sin(p) on hd/2.
    sh = TINY.replace(qk_norm=False, eps=0.0)
    ws = _tiny_weights(sh)[0]
    ws["attn_norm"] = np.ones(sh.hidden)
    wqkv = ws["w_qkv"].copy()
    k0 = sh.nq * sh.head_dim
    wqkv[k0:k0 + sh.nkv * sh.head_dim] = 0.0
    for j in range(sh.nkv):
        wqkv[k0 + j * sh.head_dim] = 1.0 / sh.hidden
    ws["w_qkv"] = wqkv
    kc, vc = _nan_caches(sh)
    start, n = 11, 5
    kc[:, :, :start] = 0.0
    vc[:, :, :start] = 0.0
    oracle.prefill_layer(sh, ws, 0, np.full((n, sh.hidden), 2.0), start, kc, vc)
    for t in range(n):
        p = start + t
        expect = np.zeros(sh.head_dim)
        expect[0], expect[sh.head_dim // 2] = math.cos(p), math.sin(p)
        for j in range(sh.nkv):
            np.testing.assert_allclose(kc[0, j, p], expect, atol=1e-15)


def _qkv_weights_from_vectors(q_pre, k_pre, v_pre, hidden):
    """Fused QKV rows that map the all-ones normed row onto the given vectors:
    every column of row d holds vec[d] / H, so the row's dot product with
    H ones is vec[d] (exact for the dyadic values used here)."""
    rows = [np.full(hidden, c / hidden) for vecs in (q_pre, k_pre, v_pre)
            for head in vecs for c in head]
    return np.array(rows, dtype=np.float64)


@pytest.mark.parametrize("case", _golden()["qk_norm_rope"])
def test_qk_norm_rope_hand_case(case):
    # the query and key of one token at a known position, through the layer's
    # own projection, per-head QK-norm and RoPE (qkv_rows), and the K/V values
    # the layer leaves in the cache slot of that position (prefill_layer)
    hd, nq, nkv = case["head_dim"], case["n_q_heads"], case["n_kv_heads"]
    H = 4
    sh = synth.Shape("qk-hand", hidden=H, inter=4, nq=nq, nkv=nkv, head_dim=hd, qk_norm=True,
                     eps=case["eps"], theta=case["theta"], n_tokens=1, start=case["position"],
                     max_seq=8, dtype="f32")
    w = {"attn_norm": np.ones(H), "q_norm": np.array(case["q_gain"]),
         "k_norm": np.array(case["k_gain"]),
         "w_qkv": _qkv_weights_from_vectors(case["q_pre"], case["k_pre"], case["v_pre"], H),
         "w_o": np.zeros((H, nq * hd)), "ffn_norm": np.ones(H),
         "w_gate_up": np.zeros((2 * sh.inter, H)), "w_down": np.zeros((H, sh.inter))}
    x = np.ones((1, H))
    p = case["position"]
    q, k, v = oracle.qkv_rows(sh, w, x, np.array([p]))
    exp_q = np.array([_eval(h) for h in case["expected_q"]])
    exp_k = np.array([_eval(h) for h in case["expected_k"]])
    exp_v = np.array([_eval(h) for h in case["expected_v"]])
    np.testing.assert_allclose(q[0], exp_q, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(k[0], exp_k, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(v[0], exp_v, rtol=0, atol=0)
    kc = np.zeros((1, nkv, sh.max_seq, hd))
    vc = np.zeros((1, nkv, sh.max_seq, hd))
    oracle.prefill_layer(sh, w, 0, x, p, kc, vc)
    np.testing.assert_allclose(kc[0, :, p], exp_k, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(vc[0, :, p], exp_v, rtol=0, atol=0)


@pytest.mark.parametrize("start", [5, 7])
def test_layer_scores_follow_normed_roped_query(start):
    # The query side of the layer, end to end.  The hidden row is constant, so
    # with a unit attention gain and eps 0 the normed row is all ones.  W_q
    # makes head 0's query e_0 and head 1's 3*e_1 before QK-norm: per head the
    # norm gives sqrt(hd)*g_q[0]*e_0 and sqrt(hd)*g_q[1]*e_1.  The cache slots
    # u < p hold K_u = R_u(e_0 + e_1) and one-hot V_u = e_u, so after RoPE the
    # score of head h against slot u is g_q[h] * cos((p-u) * theta_h) (the
    # 1/sqrt(hd) scale cancels the sqrt(hd)).  The token's own key is
    # sqrt(hd)*g_k[2]*e_2 roped at p, orthogonal to both queries (score 0),
    # and its value is 0.  W_o = identity and W_down = 0, so the output row is
    # the input plus, for head h, the softmax weight of slot u on hidden dim
    # h*hd + u.  Non-uniform gains make a swapped q/k gain, a norm taken after
    # RoPE or over all heads at once, and an unrotated or rescaled query change
    # the result.
    hd, nq, nkv, H, theta = 8, 2, 1, 16, 1e4
    p = start
    sh = synth.Shape("q-path", hidden=H, inter=4, nq=nq, nkv=nkv, head_dim=hd, qk_norm=True,
                     eps=0.0, theta=theta, n_tokens=1, start=p, max_seq=8, dtype="f32")
    g_q = np.array([1.5, 0.75, 1.1, 0.9, 1.2, 0.8, 1.3, 0.7])
    g_k = np.array([0.6, 1.4, 1.25, 0.95, 1.05, 0.85, 1.15, 0.65])
    q_pre = [[1.0 if d == 0 else 0.0 for d in range(hd)], [3.0 if d == 1 else 0.0 for d in range(hd)]]
    k_pre = [[1.0 if d == 2 else 0.0 for d in range(hd)]]
    v_pre = [[0.0] * hd]
    w = {"attn_norm": np.ones(H), "q_norm": g_q, "k_norm": g_k,
         "w_qkv": _qkv_weights_from_vectors(q_pre, k_pre, v_pre, H),
         "w_o": np.eye(H), "ffn_norm": np.ones(H),
         "w_gate_up": np.zeros((2 * sh.inter, H)), "w_down": np.zeros((H, sh.inter))}
    freq = [theta ** (-2.0 * i / hd) for i in range(hd // 2)]
    kc = np.full((1, nkv, sh.max_seq, hd), np.nan)
    vc = np.full((1, nkv, sh.max_seq, hd), np.nan)
    for u in range(p):
        kc[0, 0, u] = 0.0
        for i in (0, 1):
            kc[0, 0, u, i] = math.cos(u * freq[i])
            kc[0, 0, u, i + hd // 2] = math.sin(u * freq[i])
        vc[0, 0, u] = 0.0
        vc[0, 0, u, u] = 1.0
    x = np.full((1, H), 2.0)
    out = oracle.prefill_layer(sh, w, 0, x, p, kc, vc)
    expect = np.full(H, 2.0)
    for h in range(nq):
        e = [math.exp(g_q[h] * math.cos((p - u) * freq[h])) for u in range(p)]
        den = sum(e) + 1.0                      # the token's own slot: score 0, value 0
        for u in range(p):
            expect[h * hd + u] += e[u] / den
    np.testing.assert_allclose(out[0], expect, rtol=1e-14, atol=1e-14)
    # the key written at slot p: R_p(sqrt(hd) * g_k[2] * e_2)
    r = math.sqrt(hd) * g_k[2]
    kp = np.zeros(hd)
    kp[2], kp[2 + hd // 2] = r * math.cos(p * freq[2]), r * math.sin(p * freq[2])
    np.testing.assert_allclose(kc[0, 0, p], kp, rtol=1e-14, atol=1e-14)


def test_layer_value_path_running_mean():
    # Q = K = 0 makes every score 0, so attention is the plain mean of the visible
    # values; V head j is xn itself on its first hd dims; W_o copies head 0 back
    # onto hidden dims [0, hd); W_down = 0.  Token t at start 0 must then gain the
    # mean of xn[0..t] on those dims: this pins the V slice, the causal window,
    # the cache round trip and the residual add.  QK-norm is on (a zero row
    # normalises to zero), so a V that were normed as well would show here.
    sh = TINY
    ws = _tiny_weights(sh)[0]
    hd, nq, nkv, H = sh.head_dim, sh.nq, sh.nkv, sh.hidden
    wqkv = np.zeros((sh.qkv_dim, H))
    for j in range(nkv):
        for d in range(hd):
            wqkv[(nq + nkv) * hd + j * hd + d, d] = 1.0
    ws["w_qkv"] = wqkv
    wo = np.zeros((H, nq * hd))
    wo[np.arange(hd), np.arange(hd)] = 1.0
    ws["w_o"] = wo
    ws["w_down"] = np.zeros_like(ws["w_down"])
    x = np.random.default_rng(14).standard_normal((7, H))
    kc, vc = _nan_caches(sh)
    out = oracle.prefill_layer(sh, ws, 0, x, 0, kc, vc)
    xn = oracle.rms_norm(x, ws["attn_norm"], sh.eps)
    for t in range(7):
        expect = x[t].copy()
        expect[:hd] += xn[:t + 1, :hd].mean(axis=0)
        np.testing.assert_allclose(out[t], expect, rtol=1e-13, atol=1e-13)


def test_layer_ffn_gate_and_up_halves():
    # W_o = 0 and a unit W_down row map; gate row i reads xn2 dim 0, up row i reads
    # dim 1: the FFN adds silu(xn2[0]) * xn2[1] to hidden dim i for i < I.
    sh = TINY
    ws = _tiny_weights(sh)[0]
    H, I = sh.hidden, sh.inter
    ws["w_o"] = np.zeros_like(ws["w_o"])
    wgu = np.zeros((2 * I, H))
    wgu[:I, 0] = 1.0
    wgu[I:, 1] = 1.0
    ws["w_gate_up"] = wgu
    wd = np.zeros((H, I))
    wd[np.arange(I), np.arange(I)] = 1.0
    ws["w_down"] = wd
    x = np.random.default_rng(15).standard_normal((3, H))
    kc, vc = _nan_caches(sh)
    out = oracle.prefill_layer(sh, ws, 0, x, 0, kc, vc)
    xn2 = oracle.rms_norm(x, ws["ffn_norm"], sh.eps)
    add = xn2[:, 0] / (1 + np.exp(-xn2[:, 0])) * xn2[:, 1]
    expect = x.copy()
    expect[:, :I] += add[:, None]
    np.testing.assert_allclose(out, expect, rtol=1e-13, atol=1e-14)


def _run_chunked(shape, ws, x, start, mb, prefill=None):
    kc, vc = _nan_caches(shape)
    if prefill is not None:
        kc[:, :, :start], vc[:, :, :start] = prefill
    out, _ = oracle.prefill_chunk(shape, ws, x, start, mb, kc, vc)
    return out, kc, vc


def test_one_shot_chunked_and_token_by_token_agree():
    ws = _tiny_weights(TINY)
    rng = np.random.default_rng(16)
    start, n = 3, 9
    pre = (rng.standard_normal((2, 2, start, 16)), rng.standard_normal((2, 2, start, 16)))
    x = rng.standard_normal((n, TINY.hidden))
    one, k1, v1 = _run_chunked(TINY, ws, x, start, 0, pre)
    for mb in (1, 2, 4, 5):
        got, k2, v2 = _run_chunked(TINY, ws, x, start, mb, pre)
        np.testing.assert_allclose(got, one, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(k2, k1, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(v2, v1, rtol=1e-12, atol=1e-12)
        assert np.array_equal(np.isnan(k2), np.isnan(k1))


def test_row_sampling_matches_full_layer():
    ws = _tiny_weights(TINY)[0]
    x = np.random.default_rng(17).standard_normal((8, TINY.hidden))
    kc, vc = _nan_caches(TINY)
    full = oracle.prefill_layer(TINY, ws, 0, x, 0, kc, vc)
    kc, vc = _nan_caches(TINY)
    rows = np.array([0, 5, 7])
    part = oracle.prefill_layer(TINY, ws, 0, x, 0, kc, vc, rows=rows)
    np.testing.assert_allclose(part, full[rows], rtol=1e-13, atol=1e-14)


def test_head_reads_last_row_normed():
    sh = TINY
    rng = np.random.default_rng(18)
    x = rng.standard_normal((4, sh.hidden))
    g = 1 + 0.05 * rng.standard_normal(sh.hidden)
    logits = oracle.lm_head_logits(x[-1], g, 1e-5, np.eye(sh.hidden))
    ms = np.mean(x[-1] ** 2)
    np.testing.assert_allclose(logits, g * x[-1] / math.sqrt(ms + 1e-5), rtol=1e-14)


def test_sign1_layer_equals_dense_layer_of_decoded_weights():
    sh = TINY.replace(hidden=128, inter=256, nq=2, nkv=1, head_dim=64, wformat="sign1")
    w_q = synth.widen_layer(sh, synth.layer_weights(sh, 0))
    w_d = {k: (oracle.decode_sign1(*v) if isinstance(v, tuple) else v) for k, v in w_q.items()}
    x = np.random.default_rng(19).standard_normal((3, sh.hidden))
    kc, vc = _nan_caches(sh)
    a = oracle.prefill_layer(sh, w_q, 0, x, 0, kc, vc)
    kc, vc = _nan_caches(sh)
    b = oracle.prefill_layer(sh, w_d, 0, x, 0, kc, vc)
    assert np.array_equal(a, b)


def test_chunk_head_runs_on_final_token_of_last_micro_batch():
    sh = TINY
    ws = _tiny_weights(sh)
    x = np.random.default_rng(20).standard_normal((7, sh.hidden))
    g = np.ones(sh.hidden)
    kc, vc = _nan_caches(sh)
    out, logits = oracle.prefill_chunk(sh, ws, x, 0, 3, kc, vc, final_gain=g,
                                       head=np.eye(sh.hidden), final_eps=0.0)
    last = out[-1]
    np.testing.assert_allclose(logits, last / math.sqrt(np.mean(last ** 2)), rtol=1e-14)


# ---------------------------------------------------------------- greedy argmax and verify tail

@pytest.mark.parametrize("case", _golden()["argmax"])
def test_argmax_hand_cases(case):
    logits = np.array([float(v) for v in case["logits"]], dtype=np.float64)
    assert int(oracle.argmax_rows(logits)) == case["expected"]


def test_argmax_rows_is_per_row_and_brute_force():
    rng = np.random.default_rng(5)
    x = rng.integers(-3, 4, size=(9, 13)).astype(np.float64)   # many ties
    got = oracle.argmax_rows(x)
    for r in range(x.shape[0]):
        best = max(x[r])
        assert got[r] == min(v for v in range(x.shape[1]) if x[r, v] == best)


@pytest.mark.parametrize("case", _golden()["verify_tail"])
def test_verify_tail_hand_cases(case):
    logits, tokens = oracle.verify_tail(np.array(case["x"]), np.array(case["gain"]),
                                        case["eps"], np.array(case["head"]))
    exp = np.array([_eval(row) for row in case["expected_logits"]])
    np.testing.assert_allclose(logits, exp, rtol=1e-15, atol=1e-15)
    assert tokens.tolist() == case["expected_tokens"]


def test_verify_tail_rows_are_normed_independently():
    # at eps = 0 a row's logits do not change when the row is scaled, whatever
    # the other rows hold; a norm over the batch (or over columns) would
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 8))
    W = rng.standard_normal((5, 8))
    g = 1 + 0.1 * rng.standard_normal(8)
    base, _ = oracle.verify_tail(x, g, 0.0, W)
    scaled = x * np.array([[1.0], [7.0], [0.25]])
    got, _ = oracle.verify_tail(scaled, g, 0.0, W)
    np.testing.assert_allclose(got, base, rtol=1e-12)


# ---------------------------------------------------------------- fp16 KV cache

@pytest.mark.parametrize("case", _golden()["f16_cache"])
def test_f16_cache_rounding_hand_cases(case):
    ns = dict(MATH_NS, inf=math.inf)
    x = eval(case["x"], {"__builtins__": {}}, ns)
    exp = eval(case["expected"], {"__builtins__": {}}, ns)
    sh = synth.WORKLOADS["tiny-f32"].replace(dtype="bf16", kv="f16")
    got = oracle.cache_store(sh, np.array([x, -x]))
    assert got[0] == exp and got[1] == -exp


def test_act_format_cache_is_exact():
    sh = synth.WORKLOADS["tiny-f32"]
    x = np.array([1 + 2.0 ** -40, math.pi])
    assert np.array_equal(oracle.cache_store(sh, x), x)


def test_layer_with_f16_cache_stores_rounded_keys_and_reads_them():
    # the f16-cache layer equals the exact layer run on caches whose written
    # slots are the halves of the exact ones: store rounding is the only change
    sh = synth.WORKLOADS["tiny-f32"].replace(dtype="bf16", n_tokens=6, start=3, max_seq=16)
    sh16 = sh.replace(kv="f16")
    w = synth.widen_layer(sh, synth.layer_weights(sh, 0))
    x = synth.widen(synth.hidden_input(sh), sh.dtype)
    kc, vc = synth.kv_caches(sh16)
    k16, v16 = synth.widen(kc, "f16"), synth.widen(vc, "f16")
    out16 = oracle.prefill_layer(sh16, w, 0, x, sh.start, k16, v16)
    pos = sh.start + np.arange(sh.n_tokens)
    _, k, v = oracle.qkv_rows(sh, w, x, pos)
    assert np.array_equal(k16[0][:, sh.start:sh.start + sh.n_tokens],
                          k.transpose(1, 0, 2).astype(np.float16).astype(np.float64))
    assert np.array_equal(v16[0][:, sh.start:sh.start + sh.n_tokens],
                          v.transpose(1, 0, 2).astype(np.float16).astype(np.float64))
    # the same layer with exact caches differs, but only by about the rounding
    k64, v64 = synth.widen(kc, "f16"), synth.widen(vc, "f16")
    out = oracle.prefill_layer(sh, w, 0, x, sh.start, k64, v64)
    assert not np.array_equal(out, out16)
    assert np.abs(out - out16).max() <= 1e-2 * np.abs(out).max()
