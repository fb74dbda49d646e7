"""Pins of the oracle's LM head (paperlayer.ai summary of arXiv 2604.18396v3, section 4
"Inference with Seamless Exit": after the last layer the original LM head produces the logits,
from the final-normed state). Closed forms: a constant state c*1 has rms |c|, so the final
RMSNorm maps element j to sign(c)*|c|/sqrt(c^2 + eps) * g_j (rounded to fp16); a head row that
is a one-hot e_j scaled by a then gives logit a * x_j. Untied models must read lm_head, tied
models the embedding."""

import math

import numpy as np

from oracle import river_oracle as O

D, V, EPS = 8, 6, 1e-5


def _cfg():
    return {"L": 1, "d": D, "H": 1, "Hkv": 1, "D": D, "F": 8, "V": V, "eps": EPS,
            "theta": 10000.0, "group": 8, "entry": 1}


def _weights(head, embed, gains):
    return {"embed": embed.astype(np.float16),
            "lm_head": None if head is None else head.astype(np.float16),
            "final_norm": gains.astype(np.float16), "layers": [None]}


def _one_hot_rows(cols, scale):
    m = np.zeros((V, D), np.float64)
    for v, (j, a) in enumerate(zip(cols, scale)):
        m[v, j] = a
    return m


def test_constant_state_one_hot_head_closed_form():
    gains = np.array([1.0, 0.5, 2.0, -1.0, 0.25, 3.0, 1.5, -0.75])
    cols = [3, 0, 5, 5, 7, 1]
    scale = [1.0, 2.0, -1.0, 0.5, 4.0, 1.0]
    head = _one_hot_rows(cols, scale)
    embed = np.full((V, D), 0.01)  # must not be used: the model is untied
    orc = O.RiverOracle(_cfg(), _weights(head, embed, gains), layers=[])
    for c in (0.75, -2.0, 1e-3):
        h = np.full(D, c, np.float16)
        cc = float(np.float16(c))
        x = [float(np.float16(math.copysign(abs(cc) / math.sqrt(cc * cc + EPS), cc) * g)) for g in gains]
        want = [a * x[j] for j, a in zip(cols, scale)]
        got = orc.head_logits(h)
        assert np.allclose(got, want, rtol=0, atol=1e-12), (c, got, want)


def test_untied_reads_lm_head_tied_reads_embedding():
    gains = np.ones(D)
    rng = np.random.default_rng(0)
    embed = rng.normal(0, 0.5, (V, D))
    head = _one_hot_rows([0, 1, 2, 3, 4, 5], [1, 1, 1, 1, 1, 1])
    h = np.float16(rng.normal(0, 1, D))
    untied = O.RiverOracle(_cfg(), _weights(head, embed, gains), layers=[])
    tied = O.RiverOracle(_cfg(), _weights(None, embed, gains), layers=[])
    x = O.rmsnorm(h, gains.astype(np.float16), EPS).astype(np.float64)
    # untied: one-hot rows pick x_0..x_5
    assert np.array_equal(untied.head_logits(h), x[:V])
    # tied: the logits are the embedding rows against x (dot products done here in fp64 by hand)
    e16 = embed.astype(np.float16).astype(np.float64)
    want = [sum(e16[v, j] * x[j] for j in range(D)) for v in range(V)]
    assert np.allclose(tied.head_logits(h), want, rtol=0, atol=1e-12)
    assert not np.allclose(tied.head_logits(h), untied.head_logits(h))


def test_final_norm_is_applied_and_scale_invariant():
    """The logits of h and of k*h agree (RMSNorm removes the scale, up to eps and fp16
    rounding), and a zero gain zeroes that coordinate's contribution."""
    gains = np.array([1.0, 1.0, 0.0, 1.0, 1.0, 1.0, 1.0, 1.0])
    head = _one_hot_rows([0, 1, 2, 3, 4, 5], [1, 1, 1, 1, 1, 1])
    orc = O.RiverOracle(_cfg(), _weights(head, np.zeros((V, D)), gains), layers=[])
    h = np.array([0.5, -1.0, 2.0, 0.25, -0.75, 1.5, 1.0, -0.5], np.float16)
    a = orc.head_logits(h)
    b = orc.head_logits((h.astype(np.float64) * 4.0).astype(np.float16))
    assert a[2] == 0.0 and b[2] == 0.0
    assert np.allclose(a, b, rtol=2e-3, atol=0)
    rms = math.sqrt(float(np.mean(h.astype(np.float64) ** 2)) + EPS)
    assert abs(a[1] - (-1.0 / rms)) < 1e-3
