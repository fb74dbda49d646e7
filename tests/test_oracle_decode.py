"""Pins of the oracle's block, prefill and decode against identities the method fixes,
and of one block against a pure-Python brute force (no GPU)."""

import math

import numpy as np
import pytest
import torch

from oracle import river_oracle as O
from token_level_early_amd import configs, synth

TINY = configs.model_cfg(configs.TINY)


@pytest.fixture(scope="module")
def tiny_w():
    return synth.to_numpy(synth.weights(TINY, seed=0, device="cpu"))


@pytest.fixture(scope="module")
def tiny_model(tiny_w):
    return O.RiverOracle(TINY, tiny_w)


def _prompt(B, P, seed=0):
    return synth.prompt(TINY, B, P, seed=seed).numpy()


def _run(model, B, P, steps, forced=None, tau=None, prefill_exit=None, Tmax=None, seed=0,
         gpu_exit=None):
    kv = model.new_kv(B, Tmax or (P + steps))
    toks = _prompt(B, P, seed)
    if prefill_exit is None and tau is None:
        prefill_exit = model.cfg["L"]  # forced decode schedules start from a full-depth prefill
    pre = model.prefill(kv, toks, prefill_exit=prefill_exit,
                        tau=tau if prefill_exit is None else None)
    cur = pre["tokens"]
    outs = []
    for s in range(steps):
        f = None if forced is None else forced[s]
        g = None if gpu_exit is None else gpu_exit[s]
        r = model.decode_step(kv, cur, forced_exit=f, tau=tau, gpu_exit=g)
        outs.append(r)
        cur = r["tokens"]
    return pre, outs, kv


# ---------------------------------------------------------------- brute-force block

def _bf_block(cfg, W, norms, h_in, pos, Kc, Vc):
    """One Llama block written with explicit Python loops over indices (fp64 math,
    fp16 rounding through np.float16 on scalars). Kc/Vc: nested lists [Hkv][T][D]."""
    r16 = lambda x: float(np.float16(x))  # noqa: E731
    H, Hkv, D, eps, theta = cfg["H"], cfg["Hkv"], cfg["D"], cfg["eps"], cfg["theta"]
    d = len(h_in)

    def norm(x, w):
        ms = sum(v * v for v in x) / len(x)
        inv = 1.0 / math.sqrt(ms + eps)
        return [r16(x[i] * inv * w[i]) for i in range(len(x))]

    def mv(M, x):
        return [sum(M[n][k] * x[k] for k in range(len(x))) for n in range(len(M))]

    def rope(vec, nh):
        out = list(vec)
        for h in range(nh):
            for i in range(D // 2):
                ang = pos * theta ** (-2.0 * i / D)
                a, b = vec[h * D + i], vec[h * D + i + D // 2]
                out[h * D + i] = r16(a * math.cos(ang) - b * math.sin(ang))
                out[h * D + i + D // 2] = r16(b * math.cos(ang) + a * math.sin(ang))
        return out

    a = norm(h_in, norms["attn_norm"])
    q = rope([r16(v) for v in mv(W["wq"], a)], H)
    k = rope([r16(v) for v in mv(W["wk"], a)], Hkv)
    v = [r16(x) for x in mv(W["wv"], a)]
    for j in range(Hkv):
        Kc[j].append(k[j * D:(j + 1) * D])
        Vc[j].append(v[j * D:(j + 1) * D])
    o = []
    for h in range(H):
        j = h // (H // Hkv)
        T = len(Kc[j])
        sc = [sum(q[h * D + i] * Kc[j][t][i] for i in range(D)) / math.sqrt(D) for t in range(T)]
        m = max(sc)
        w = [math.exp(s - m) for s in sc]
        z = sum(w)
        o += [r16(sum(w[t] * Vc[j][t][i] for t in range(T)) / z) for i in range(D)]
    y = mv(W["wo"], o)
    hm = [r16(h_in[i] + r16(y[i])) for i in range(d)]
    mm = norm(hm, norms["mlp_norm"])
    g = [r16(x) for x in mv(W["w_gate"], mm)]
    u = [r16(x) for x in mv(W["w_up"], mm)]
    a2 = [r16(g[f] / (1 + math.exp(-g[f])) * u[f]) for f in range(len(g))]
    y2 = mv(W["w_down"], a2)
    return [r16(hm[i] + r16(y2[i])) for i in range(d)]


def test_block_matches_python_loops():
    cfg = dict(H=2, Hkv=1, D=4, eps=1e-5, theta=10000.0)
    d, F, T0 = 8, 6, 3
    rng = np.random.default_rng(7)
    sh = {"wq": (8, d), "wk": (4, d), "wv": (4, d), "wo": (d, 8), "w_gate": (F, d),
          "w_up": (F, d), "w_down": (d, F)}
    W16 = {k: (rng.standard_normal(s) * 0.3).astype(np.float16) for k, s in sh.items()}
    norms = {"attn_norm": (1 + 0.1 * rng.standard_normal(d)).astype(np.float16),
             "mlp_norm": (1 + 0.1 * rng.standard_normal(d)).astype(np.float16)}
    h_in = rng.standard_normal(d).astype(np.float16)
    K0 = rng.standard_normal((1, T0, 4)).astype(np.float16)
    V0 = rng.standard_normal((1, T0, 4)).astype(np.float16)
    Kc = np.zeros((1, 8, 4), np.float16)
    Vc = np.zeros((1, 8, 4), np.float16)
    Kc[:, :T0], Vc[:, :T0] = K0, V0
    W64 = {k: v.astype(np.float64) for k, v in W16.items()}
    out = O.block_decode(cfg, W64, norms, h_in, T0, Kc, Vc)
    want = _bf_block(cfg, {k: v.astype(np.float64).tolist() for k, v in W16.items()},
                     {k: v.astype(np.float64).tolist() for k, v in norms.items()},
                     h_in.astype(np.float64).tolist(), T0,
                     [K0[0].astype(np.float64).tolist()], [V0[0].astype(np.float64).tolist()])
    # same arithmetic up to fp64 summation order -> equal up to one fp16 rounding flip
    assert np.allclose(out.astype(np.float64), want, rtol=2 ** -10, atol=1e-4)
    assert (Kc[0, T0] != 0).any() and (Kc[0, T0 + 1] == 0).all()


def test_block_residual_identity_when_projections_are_zero(tiny_w):
    rng = np.random.default_rng(8)
    lw = tiny_w["layers"][0]
    W = {m: lw[m].astype(np.float64) for m in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")}
    W["wo"] = np.zeros_like(W["wo"])
    W["w_down"] = np.zeros_like(W["w_down"])
    h = rng.standard_normal(TINY["d"]).astype(np.float16)
    K = np.zeros((TINY["Hkv"], 4, TINY["D"]), np.float16)
    V = np.zeros_like(K)
    out = O.block_decode(TINY, W, {"attn_norm": lw["attn_norm"], "mlp_norm": lw["mlp_norm"]},
                         h, 2, K, V)
    assert (out == h).all()
    assert (K[:, 2] != 0).any() and (V[:, 2] != 0).any()  # KV still produced


# ---------------------------------------------------------------- exit-rule identities

def test_tau_above_one_never_exits_and_equals_full_backbone(tiny_model):
    L = TINY["L"]
    _, a, kva = _run(tiny_model, 1, 8, 4, tau=1.5)
    _, b, kvb = _run(tiny_model, 1, 8, 4, forced=[[L]] * 4)
    for ra, rb in zip(a, b):
        assert ra["exit_layer"].tolist() == [L]
        assert (ra["hs"] == rb["hs"]).all()
        assert (ra["logits"] == rb["logits"]).all()
        assert (ra["tokens"] == rb["tokens"]).all()
        assert np.isfinite(ra["sim"][0, : L - 1]).all() and np.isnan(ra["sim"][0, L - 1])
    assert (kva.K == kvb.K).all() and (kva.V == kvb.V).all()


def test_tau_below_minus_one_exits_at_entry(tiny_w):
    for entry in (1, 2):
        m = O.RiverOracle(dict(TINY, entry=entry), tiny_w)
        _, outs, _ = _run(m, 1, 8, 3, tau=-1.5)
        assert all(r["exit_layer"].tolist() == [entry] for r in outs)
        # nothing is tested before the entry layer or after the exit
        assert all(np.isnan(r["sim"][0, : entry - 1]).all() for r in outs)
        assert all(np.isnan(r["sim"][0, entry:]).all() for r in outs)


def test_forced_schedule_sets_exit_layer_and_uses_river(tiny_model):
    L = TINY["L"]
    _, a, kva = _run(tiny_model, 1, 8, 2, forced=[[1], [1]])
    _, b, kvb = _run(tiny_model, 1, 8, 2, forced=[[L], [L]])
    assert a[0]["exit_layer"].tolist() == [1]
    # layer 1 ran on the backbone in both runs; layer 2 on the river only in run a
    assert (a[0]["hs"][1] == b[0]["hs"][1]).all()
    assert (a[0]["hs"][2] != b[0]["hs"][2]).any()
    P = 8
    assert (kva.K[0, 0, :, P] == kvb.K[0, 0, :, P]).all()
    assert (kva.K[1, 0, :, P] != kvb.K[1, 0, :, P]).any()


def test_representable_weights_river_equals_backbone():
    w = synth.to_numpy(synth.representable_weights(TINY, seed=1))
    m = O.RiverOracle(TINY, w)
    L = TINY["L"]
    _, a, kva = _run(m, 1, 8, 3, forced=[[1]] * 3)
    _, b, kvb = _run(m, 1, 8, 3, forced=[[L]] * 3)
    for ra, rb in zip(a, b):
        assert (ra["hs"] == rb["hs"]).all()
        assert (ra["logits"] == rb["logits"]).all()
    assert (kva.K == kvb.K).all() and (kva.V == kvb.V).all()


def test_kv_slots_written_exactly_once_under_random_schedules(tiny_model):
    L, P, S = TINY["L"], 6, 5
    rng = np.random.default_rng(9)
    for trial in range(3):
        sched = rng.integers(1, L + 1, size=(S, 2))
        _, _, kv = _run(tiny_model, 2, P, S, forced=sched, Tmax=P + S + 3, seed=trial)
        assert (kv.count[:, :, : P + S] == 1).all()
        assert (kv.count[:, :, P + S:] == 0).all()
        assert (kv.K[:, :, :, : P + S] != 0).any(axis=-1).all()


def test_margin_rule_takes_gpu_decision_only_inside_margin(tiny_model):
    # record s(1) of the first decode step, then set tau exactly there
    _, outs, _ = _run(tiny_model, 1, 8, 1, tau=1.5)
    s1 = outs[0]["sim"][0, 0]
    _, o_exit, _ = _run(tiny_model, 1, 8, 1, tau=s1, gpu_exit=[[1]])
    _, o_stay, _ = _run(tiny_model, 1, 8, 1, tau=s1, gpu_exit=[[TINY["L"]]])
    assert o_exit[0]["exit_layer"][0] == 1
    assert o_stay[0]["exit_layer"][0] != 1
    # outside the margin the GPU's decision is ignored
    _, o_far, _ = _run(tiny_model, 1, 8, 1, tau=s1 - 0.01, gpu_exit=[[TINY["L"]]])
    assert o_far[0]["exit_layer"][0] == 1


def test_batch_rows_are_independent(tiny_model):
    _, both, _ = _run(tiny_model, 2, 6, 2, forced=[[2, 3], [3, 1]], seed=3)
    toks = _prompt(2, 6, seed=3)
    for b in range(2):
        kv = tiny_model.new_kv(1, 8)
        pre = tiny_model.prefill(kv, toks[b:b + 1], prefill_exit=TINY["L"])
        cur = pre["tokens"]
        for s, fe in enumerate(([2, 3], [3, 1])):
            r = tiny_model.decode_step(kv, cur, forced_exit=[fe[b]])
            assert (r["hs"][:, 0] == both[s]["hs"][:, b]).all()
            assert r["exit_layer"][0] == fe[b]
            cur = r["tokens"]


# ---------------------------------------------------------------- prefill

def test_prefill_then_decode_matches_longer_prefill(tiny_model):
    L, P = TINY["L"], 9
    toks = _prompt(1, P + 1, seed=5)
    kv1 = tiny_model.new_kv(1, P + 1)
    tiny_model.prefill(kv1, toks[:, :P], prefill_exit=L)
    r = tiny_model.decode_step(kv1, toks[:, P], forced_exit=[L])
    kv2 = tiny_model.new_kv(1, P + 1)
    full = tiny_model.prefill(kv2, toks, prefill_exit=L)
    rms = np.sqrt(np.mean(full["logits"] ** 2))
    assert np.max(np.abs(r["logits"] - full["logits"])) / rms < 1e-2
    assert np.max(np.abs(kv1.K.astype(float) - kv2.K.astype(float))) < 2e-2


def test_prefill_sequence_exit_uses_min_over_tokens(tiny_model):
    P = 8
    toks = _prompt(1, P, seed=6)
    kv = tiny_model.new_kv(1, P)
    ref = tiny_model.prefill(kv, toks, tau=1.5, keep_hidden=True)
    assert ref["seq_exit"][0] == TINY["L"]
    s_tok = [O.cosine(ref["hs"][0, 0, t], ref["hs"][1, 0, t]) for t in range(P)]
    assert ref["min_sim"][0, 0] == pytest.approx(min(s_tok), abs=1e-15)
    lo, hi = min(s_tok), max(s_tok)
    assert hi - lo > 1e-3
    # tau just under the minimum: the whole sequence exits after layer 1
    r = tiny_model.prefill(tiny_model.new_kv(1, P), toks, tau=lo - 1e-4)
    assert r["seq_exit"][0] == 1
    # tau between min and max: some tokens would exit, the latest one keeps the sequence
    r = tiny_model.prefill(tiny_model.new_kv(1, P), toks, tau=(lo + hi) / 2)
    assert r["seq_exit"][0] != 1


def test_forced_zero_runs_every_block_on_the_river():
    """Forced exit 0 (the pages' all-int4 "Full Quantization" comparator, paperlayer summary
    §5): no backbone block. With int4-representable weights the river is the backbone exactly,
    so the result equals the full-backbone run bit for bit; with ordinary weights block 1
    already differs from a run that exits after backbone block 1."""
    L = TINY["L"]
    w = synth.to_numpy(synth.representable_weights(TINY, seed=1))
    m = O.RiverOracle(TINY, w)
    _, a, kva = _run(m, 1, 8, 3, forced=[[0]] * 3)
    _, b, kvb = _run(m, 1, 8, 3, forced=[[L]] * 3)
    for ra, rb in zip(a, b):
        assert ra["exit_layer"][0] == 0
        assert (ra["hs"] == rb["hs"]).all() and (ra["logits"] == rb["logits"]).all()
    assert (kva.K == kvb.K).all() and (kva.V == kvb.V).all()

    m2 = O.RiverOracle(TINY, synth.to_numpy(synth.weights(TINY, seed=0)))
    _, z, kvz = _run(m2, 1, 8, 1, forced=[[0]])
    _, one, kv1 = _run(m2, 1, 8, 1, forced=[[1]])
    assert (z[0]["hs"][0] == one[0]["hs"][0]).all()        # same embedding row
    assert (z[0]["hs"][1] != one[0]["hs"][1]).any()        # block 1: river vs backbone
    assert (kvz.K[0, 0, :, 8] != kv1.K[0, 0, :, 8]).any()  # its K slot at the decode position
    assert (kvz.count == kv1.count).all()                  # same slots written once
