"""Pins of the oracle's primitives against closed forms, hand-derived fixtures,
invariants and pure-Python brute force (no GPU)."""

import json
import math
import os

import numpy as np
import pytest

from oracle import river_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- cosine (exit test)

def test_cosine_closed_forms():
    f = np.float16
    assert O.cosine(np.array([3, 4], f), np.array([4, 3], f)) == pytest.approx(24 / 25, abs=1e-15)
    assert O.cosine(np.array([1, 2, 2], f), np.array([2, 1, 2], f)) == pytest.approx(8 / 9, abs=1e-15)
    a = np.array([0.5, -1.25, 2.0, 3.0], f)
    assert O.cosine(a, a) == pytest.approx(1.0, abs=1e-15)
    assert O.cosine(a, -a) == pytest.approx(-1.0, abs=1e-15)
    assert O.cosine(np.array([1, 0, 0], f), np.array([0, 5, 0], f)) == 0.0
    # invariant under positive scaling of either argument, not under negation
    b = np.array([1.5, 0.25, -2.0, 1.0], f)
    assert O.cosine(a, b) == pytest.approx(O.cosine(2 * a, b), abs=1e-15)
    assert O.cosine(a, b) == pytest.approx(-O.cosine(-a, b), abs=1e-15)
    # symmetric
    assert O.cosine(a, b) == pytest.approx(O.cosine(b, a), abs=1e-15)


def test_cosine_zero_norm_is_zero():
    z = np.zeros(4, np.float16)
    assert O.cosine(z, np.ones(4, np.float16)) == 0.0
    assert O.cosine(np.ones(4, np.float16), z) == 0.0


def test_cosine_uses_input_and_output_not_difference():
    # h_out = h_in + small residual update -> similarity close to 1; a large update
    # orthogonal to h_in -> similarity 1/sqrt(1 + r^2) with r the update/h_in norm ratio.
    h = np.array([1, 0, 0, 0], np.float16)
    upd = np.array([0, 3, 0, 4], np.float16)  # norm 5
    assert O.cosine(h, h + upd) == pytest.approx(1 / math.sqrt(26), abs=1e-12)


# ---------------------------------------------------------------- quantiser

def test_quant_hand_example():
    g = _gold("quant_hand_example.json")
    W = np.array([g["w_fp16"]], np.float16)
    q, s = O.quantize_w4(W, g["group"])
    assert float(s[0, 0]) == g["scale_fp16"]
    assert q[0].tolist() == g["q"]
    assert O.pack_nibbles(q)[0].tolist() == g["packed"]


def test_quant_uses_abs_max_of_negative_entries():
    # amax comes from -1.4 (a signed max would pick 0.2): s = fp16(fp32(1.4)/7) = fp16(0.2)
    W = np.array([[0.2, -1.4, 0.7, 0.0]], np.float16)
    q, s = O.quantize_w4(W, 4)
    # by hand: fp16(1.4) = 1.400390625, /7 = 0.2000558 -> fp16 grid 2^-13 -> 0.2000732421875;
    # 0.199951171875/s = 0.9994 -> 1, 0.7001953125/s = 3.4997 -> 3
    assert float(s[0, 0]) == 0.2000732421875
    assert q[0].tolist() == [1, -7, 3, 0]


def test_nibble_order_and_padding():
    q = np.array([[1, -2, 7]], np.int8)  # u = 9, 6, 15, pad 8
    p = O.pack_nibbles(q)
    assert p.tolist() == [[0x69, 0x8F]]
    assert O.unpack_nibbles(p, 3).tolist() == q.tolist()
    q2 = np.array([[-8, 7, 0, -1]], np.int8)  # u = 0, 15, 8, 7
    assert O.pack_nibbles(q2).tolist() == [[0xF0, 0x78]]


def test_zero_group_gives_zero_scale_and_code_8():
    W = np.zeros((2, 8), np.float16)
    W[1, 4:] = np.float16(0.5)
    q, s = O.quantize_w4(W, 4)
    assert s[0].tolist() == [0.0, 0.0] and s[1, 0] == 0.0
    assert (q[0] == 0).all() and (q[1, :4] == 0).all()
    p = O.pack_nibbles(q)
    assert (p[0] == 0x88).all()


def test_quant_round_trip_bound_and_range():
    rng = np.random.default_rng(1)
    W = (rng.standard_normal((64, 256)) * 0.02).astype(np.float16)
    for g in (64, 128):
        q, s = O.quantize_w4(W, g)
        Wh = O.dequantize_w4(q, s, g)
        srep = np.repeat(s.astype(np.float64), g, axis=1)
        err = np.abs(W.astype(np.float64) - Wh)
        assert (err <= 0.5 * srep * (1 + 1e-6)).all()
        assert q.min() >= -7 and q.max() <= 7          # absmax/7 scale never clips
        assert (np.abs(q).max(axis=1) == 7).all()       # the abs-max entry maps to +-7


def test_quant_groups_run_along_k_and_ragged_tail():
    # K = 10, group 4 -> groups [0,4), [4,8), [8,10): the short last group has its own scale
    W = np.zeros((2, 10), np.float16)
    W[0, :8] = np.float16(0.07)
    W[0, 8:] = np.float16(1.4)
    W[1, :] = np.float16(0.7)
    q, s = O.quantize_w4(W, 4)
    assert s.shape == (2, 3)
    s07 = float(np.float16(np.float32(np.float16(0.07)) / np.float32(7)))
    s14 = float(np.float16(np.float32(np.float16(1.4)) / np.float32(7)))
    assert s[0].tolist() == [s07, s07, s14]
    assert (q[0] == 7).all() and (q[1] == 7).all()


def test_representable_weights_reproduced_exactly():
    rng = np.random.default_rng(2)
    q0 = rng.integers(-7, 8, size=(16, 128))
    q0[:, ::64] = 7  # one |q| = 7 per group of 64
    W = (q0 * 2.0 ** -8).astype(np.float16)
    q, s = O.quantize_w4(W, 64)
    assert (s == np.float16(2.0 ** -8)).all()
    assert (q == q0).all()
    assert (O.dequantize_w4(q, s, 64) == W.astype(np.float64)).all()


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_closed_forms():
    eps = 1e-5
    # (3, 4): mean square 12.5
    out = O.rmsnorm(np.array([3, 4], np.float16), np.array([1, 1], np.float16), eps)
    want = np.array([3, 4]) / math.sqrt(12.5 + eps)
    assert np.allclose(out.astype(np.float64), want, rtol=2 ** -11)
    # constant vector c*1 with gains w -> w * c / sqrt(c^2 + eps), sign kept
    w = np.array([0.5, 1.5, -2.0, 1.0], np.float16)
    for c in (-3.0, 0.25):
        out = O.rmsnorm(np.full(4, c, np.float16), w, eps)
        want = w.astype(np.float64) * c / math.sqrt(c * c + eps)
        assert np.allclose(out.astype(np.float64), want, rtol=2 ** -11)
    # rows are normalised independently (last axis)
    X = np.array([[3, 4], [30, 40]], np.float16)
    out = O.rmsnorm(X, np.ones(2, np.float16), eps)
    assert np.allclose(out[0].astype(float), out[1].astype(float), rtol=2 ** -10)


# ---------------------------------------------------------------- RoPE

def test_rope_hand_example():
    g = _gold("rope_hand_example.json")
    c, s = O.rope_cos_sin(g["pos"], g["D"], g["theta"])
    for x, want in zip(g["inputs"], g["outputs_fp64"]):
        out = O.apply_rope(np.array(x, np.float16), c, s)
        assert np.allclose(out.astype(np.float64), want, atol=2 ** -11)


def test_rope_identity_at_zero_norm_and_relative_position():
    rng = np.random.default_rng(3)
    D, theta = 64, 10000.0
    x = rng.standard_normal((3, D)).astype(np.float16)
    c, s = O.rope_cos_sin(0, D, theta)
    assert (O.apply_rope(x, c, s) == x).all()
    c, s = O.rope_cos_sin(37, D, theta)
    y = O.apply_rope(x, c, s)
    assert np.allclose(np.linalg.norm(y.astype(float), axis=1), np.linalg.norm(x.astype(float), axis=1),
                       rtol=2e-3)
    # q.k depends only on the position difference
    q, k = x[0], x[1]

    def dot_at(m, n):
        cm, sm = O.rope_cos_sin(m, D, theta)
        cn, sn = O.rope_cos_sin(n, D, theta)
        return float(O.apply_rope(q, cm, sm).astype(float) @ O.apply_rope(k, cn, sn).astype(float))

    assert dot_at(5, 2) == pytest.approx(dot_at(105, 102), abs=2e-2)
    assert dot_at(5, 2) != pytest.approx(dot_at(2, 5), abs=1e-3)


# ---------------------------------------------------------------- attention

def _attn_bruteforce(q, K, V):
    """Pure-Python fp64 softmax attention for one head: loops, math.exp."""
    T, D = len(K), len(q)
    sc = [sum(float(q[i]) * float(K[t][i]) for i in range(D)) / math.sqrt(D) for t in range(T)]
    m = max(sc)
    w = [math.exp(x - m) for x in sc]
    z = sum(w)
    return [sum(w[t] * float(V[t][i]) for t in range(T)) / z for i in range(D)]


def test_attention_bruteforce_small_T():
    rng = np.random.default_rng(4)
    H, Hkv, D = 4, 2, 8
    for T in (1, 2, 5, 8):
        q = rng.standard_normal((H, D)).astype(np.float16)
        K = rng.standard_normal((Hkv, T, D)).astype(np.float16)
        V = rng.standard_normal((Hkv, T, D)).astype(np.float16)
        o = O.decode_attention(q, K, V)
        for h in range(H):
            want = _attn_bruteforce(q[h], K[h // 2], V[h // 2])
            assert np.allclose(o[h].astype(float), want, atol=2e-3, rtol=2 ** -10)


def test_attention_special_cases():
    rng = np.random.default_rng(5)
    H, Hkv, D, T = 4, 2, 16, 6
    q = rng.standard_normal((H, D)).astype(np.float16)
    V = rng.standard_normal((Hkv, T, D)).astype(np.float16)
    # T = 1 -> o = v
    o = O.decode_attention(q, rng.standard_normal((Hkv, 1, D)).astype(np.float16), V[:, :1])
    assert (o[0] == V[0, 0]).all() and (o[3] == V[1, 0]).all()
    # identical keys -> mean of V
    K = np.repeat(rng.standard_normal((Hkv, 1, D)).astype(np.float16), T, axis=1)
    o = O.decode_attention(q, K, V)
    assert np.allclose(o[1].astype(float), V[0].astype(float).mean(0), atol=2e-3)
    # one dominant logit -> that token's value
    K = np.zeros((Hkv, T, D), np.float16)
    K[:, 3, :] = np.float16(8.0) * np.sign(q[0]).astype(np.float16)
    q2 = np.repeat(np.sign(q[:1]).astype(np.float16), H, axis=0)
    o = O.decode_attention(q2, K, V)
    assert np.allclose(o[0].astype(float), V[0, 3].astype(float), atol=1e-3)


def test_gqa_head_mapping():
    # V of kv head j is the constant j+1: query head h must read kv head h // (H/Hkv)
    H, Hkv, D, T = 8, 2, 4, 3
    q = np.ones((H, D), np.float16)
    K = np.zeros((Hkv, T, D), np.float16)
    V = np.stack([np.full((T, D), j + 1, np.float16) for j in range(Hkv)])
    o = O.decode_attention(q, K, V)
    assert [float(o[h, 0]) for h in range(H)] == [1, 1, 1, 1, 2, 2, 2, 2]


def test_causal_attention_matches_decode_rows():
    rng = np.random.default_rng(6)
    P, H, Hkv, D = 7, 4, 2, 8
    Q = rng.standard_normal((P, H, D)).astype(np.float16)
    K = rng.standard_normal((Hkv, P, D)).astype(np.float16)
    V = rng.standard_normal((Hkv, P, D)).astype(np.float16)
    Oc = O.causal_attention(Q, K, V)
    assert (Oc[0, 0] == V[0, 0]).all()  # position 0 sees only itself
    for t in range(P):
        od = O.decode_attention(Q[t], K[:, : t + 1], V[:, : t + 1])
        assert np.allclose(Oc[t].astype(float), od.astype(float), atol=1e-3)


# ---------------------------------------------------------------- SwiGLU

def test_silu_values():
    assert O.silu(0.0) == 0.0
    assert O.silu(1.0) == pytest.approx(0.7310585786300049, abs=1e-15)
    assert O.silu(-1.0) == pytest.approx(-0.2689414213699951, abs=1e-15)


def test_argmax_lowest_index_on_ties():
    assert O.argmax_lowest([1.0, 3.0, 2.0, 3.0]) == 1
    assert O.argmax_lowest([5.0, 5.0]) == 0

