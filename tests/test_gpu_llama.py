"""GPU parity at the Llama-3.2-1B and Llama-3.1-8B shapes, through the C ABI.

1B (16 layers, d=2048, tied head): full 512-token prefill and decode steps in tau mode against
the complete CPU oracle, with tau calibrated on the GPU so that about half of the tokens exit
by layer 8.
8B (32 layers, d=4096): full 2048-token prefill and forced-schedule decode (the bench's
launch configuration); the oracle checks sampled outputs one by one: layer-1 KV of every
prompt position, per-layer slices of decode steps (the oracle block run on the GPU's own
h(l-1) and shared cache, on the route the schedule gives), and the LM head on the GPU's
final state.
"""

import numpy as np
import pytest
import torch

from oracle import river_oracle as O
from token_level_early_amd import configs, river, synth
from tests._util import TOL, TOL_E2E, f32, rel_err, top1_checked

pytestmark = pytest.mark.gpu


def _exit_frac_by(rv, c, tok, tau, steps, by):
    ex = torch.empty(steps, 1, dtype=torch.int32, device="cuda")
    rv.decode_steps(tok, sched=None, S=steps, tau=tau, exit_layer=ex)
    return float((ex.cpu().numpy() <= by).mean())


def test_llama1b_prefill_and_decode_match_oracle(decode_path):
    cfg = configs.LLAMA_1B
    c = configs.model_cfg(cfg)
    P, S = cfg["prompt"], 6
    w = synth.weights(c, seed=0, device="cuda")
    toks = synth.prompt(c, 1, P, seed=0, device="cuda")
    # calibrate tau on the GPU (bisection on the fraction of tokens exiting by layer 8)
    cal = river.River(c, w, max_seq=P + 48, max_prefill=P)
    lo, hi = 0.0, 1.0
    for _ in range(8):
        mid = (lo + hi) / 2
        pre = cal.prefill(toks, prefill_exit=c["L"])
        frac = _exit_frac_by(cal, c, pre["tokens"], f32(mid), 48, cfg["exit_by"])
        if frac > cfg["exit_frac"]:
            lo = mid
        else:
            hi = mid
    cal.close()
    tau = f32((lo + hi) / 2)
    print(f"calibrated tau = {tau:.6f}")

    orc = O.RiverOracle(c, synth.to_numpy(w))
    Tmax = P + S + 4
    rv = river.River(c, w, max_seq=Tmax, max_prefill=P)
    assert rv.decode_path() == decode_path
    kvo = orc.new_kv(1, Tmax)
    pre = rv.prefill(toks, prefill_exit=0, tau=tau, logits=True, min_sim=True)
    ge = pre["seq_exit"].cpu().numpy()
    opre = orc.prefill(kvo, toks.cpu().numpy(), tau=tau, gpu_seq_exit=ge)
    torch.cuda.synchronize()
    assert int(ge[0]) == int(opre["seq_exit"][0])
    assert rel_err(pre["logits"][0].cpu().numpy(), opre["logits"][0]) <= TOL_E2E
    assert top1_checked(int(pre["tokens"][0]), opre["logits"][0]) is not False
    kv = rv.kv_view().float().cpu().numpy()
    assert rel_err(kv[0, :, 0, :, :P], np.stack([kvo.K[0, 0, :, :P], kvo.V[0, 0, :, :P]])) <= TOL
    for l in (c["L"] // 2, c["L"] - 1):
        assert rel_err(kv[l, 0, 0, :, :P], kvo.K[l, 0, :, :P]) <= TOL_E2E, l
        assert rel_err(kv[l, 1, 0, :, :P], kvo.V[l, 0, :, :P]) <= TOL_E2E, l
    cur = pre["tokens"]
    exits = []
    for s in range(S):
        pos = P + s
        r = rv.decode_step(cur, tau=tau, logits=True, sim=True)
        g = r["exit_layer"].cpu().numpy()
        e = int(g[0])
        o = orc.decode_step(kvo, cur.cpu().numpy(), tau=tau, gpu_exit=g)
        hs16 = rv.hidden()[:, 0].cpu().numpy()
        hs = hs16.astype(np.float64)
        # end to end against the independent oracle run
        assert rel_err(hs, o["hs"][:, 0]) <= TOL_E2E, s
        assert rel_err(r["logits"][0].cpu().numpy(), o["logits"][0]) <= TOL_E2E, s
        assert top1_checked(int(r["tokens"][0]), o["logits"][0]) is not False, s
        assert e == int(o["exit_layer"][0]), s
        sim, osim = r["sim"][0].cpu().numpy(), o["sim"][0]
        assert np.array_equal(np.isnan(sim), np.isnan(osim))
        fin = ~np.isnan(osim)
        assert np.allclose(sim[fin], osim[fin], atol=5e-3), s
        # every block and the head on the GPU's own inputs (the 1e-2 bound)
        kvg = rv.kv_view()
        for l in range(1, c["L"] + 1):
            Kl = kvg[l - 1, 0, 0, :, : pos + 1].cpu().numpy().copy()
            Vl = kvg[l - 1, 1, 0, :, : pos + 1].cpu().numpy().copy()
            kg, vg = Kl[:, pos].copy(), Vl[:, pos].copy()
            out = O.block_decode(c, orc.weights_for(l - 1, l > e), orc.norms(l - 1), hs16[l - 1],
                                 pos, Kl, Vl)
            assert rel_err(hs16[l], out) <= TOL, (s, l)
            assert rel_err(kg, Kl[:, pos]) <= TOL and rel_err(vg, Vl[:, pos]) <= TOL, (s, l)
        lg = orc.head_logits(hs16[c["L"]])
        assert rel_err(r["logits"][0].cpu().numpy(), lg) <= TOL, s
        exits.append(e)
        cur = r["tokens"]
    print("exit layers", exits)
    rv.close()


@pytest.fixture(scope="module")
def llama8b():
    cfg = configs.LLAMA_8B
    c = configs.model_cfg(cfg)
    w = synth.weights(c, seed=0, device="cuda")
    return cfg, c, w


def test_llama8b_prefill_kv_layer1_matches_oracle(llama8b):
    cfg, c, w = llama8b
    P = cfg["prompt"]
    rv = river.River(c, w, max_seq=P + 8, max_prefill=P)
    toks = synth.prompt(c, 1, P, seed=0, device="cuda")
    rv.prefill(toks, prefill_exit=c["L"])
    kv = rv.kv_view()
    # oracle: layer-1 K/V of every prompt position depend only on the embedding rows
    lw = w["layers"][0]
    E = w["embed"][toks[0].long()].cpu().numpy()
    A = O.rmsnorm(E, lw["attn_norm"].cpu().numpy(), c["eps"])
    Hkv, D = c["Hkv"], c["D"]
    Kx = O.to_f16(A.astype(np.float64) @ lw["wk"].cpu().numpy().astype(np.float64).T).reshape(P, Hkv, D)
    Vx = O.to_f16(A.astype(np.float64) @ lw["wv"].cpu().numpy().astype(np.float64).T).reshape(P, Hkv, D)
    cs, sn = O.rope_cos_sin(np.arange(P), D, c["theta"])
    Kx = O.apply_rope(Kx, cs[:, None, :], sn[:, None, :])
    gk = kv[0, 0, 0, :, :P].float().cpu().numpy().transpose(1, 0, 2)
    gv = kv[0, 1, 0, :, :P].float().cpu().numpy().transpose(1, 0, 2)
    assert rel_err(gk, Kx) <= TOL
    assert rel_err(gv, Vx) <= TOL
    # nothing beyond the prompt is written
    assert float(kv[:, :, 0, :, P:].abs().max()) == 0.0
    rv.close()


def test_llama8b_decode_slices_match_oracle(llama8b, decode_path):
    cfg, c, w = llama8b
    P, W, S = cfg["prompt"], 4, 3
    L = c["L"]
    rv = river.River(c, w, max_seq=P + W + S + 4, max_prefill=P)
    assert rv.decode_path() == decode_path
    toks = synth.prompt(c, 1, P, seed=0, device="cuda")
    sched = torch.from_numpy(synth.schedule(cfg, W + S, 1, seed=0)).to("cuda")
    pre = rv.prefill(toks, prefill_exit=L)
    t = rv.decode_steps(pre["tokens"], sched=sched[:W].contiguous())
    cur = t[-1].clone()
    es = [int(x) for x in sched[W:, 0].cpu()]
    sample = sorted({1, L} | set(es) | {e + 1 for e in es if e < L})
    orc = O.RiverOracle(c, synth.to_numpy({"embed": w["embed"], "lm_head": w["lm_head"],
                                            "final_norm": w["final_norm"],
                                            "layers": [w["layers"][i] if i + 1 in sample else None
                                                       for i in range(L)]}),
                        layers=[l - 1 for l in sample])
    for s in range(S):
        e = es[s]
        pos = P + W + s
        r = rv.decode_step(cur, forced_exit=sched[W + s], logits=True)
        assert int(r["exit_layer"][0]) == e
        hs = rv.hidden()[:, 0].cpu().numpy()
        kv = rv.kv_view()
        for l in sorted({1, e, min(e + 1, L), L}):
            Kl = kv[l - 1, 0, 0, :, : pos + 1].cpu().numpy().copy()
            Vl = kv[l - 1, 1, 0, :, : pos + 1].cpu().numpy().copy()
            k_gpu, v_gpu = Kl[:, pos].copy(), Vl[:, pos].copy()
            river_path = l > e
            out = O.block_decode(c, orc.weights_for(l - 1, river_path), orc.norms(l - 1),
                                 hs[l - 1], pos, Kl, Vl)  # overwrites slot pos with the oracle's
            assert rel_err(hs[l], out) <= TOL, (s, l)
            assert rel_err(k_gpu, Kl[:, pos]) <= TOL, (s, l)
            assert rel_err(v_gpu, Vl[:, pos]) <= TOL, (s, l)
        lg = orc.head_logits(hs[L])
        assert rel_err(r["logits"][0].cpu().numpy(), lg) <= TOL
        assert top1_checked(int(r["tokens"][0]), lg) is not False
        cur = r["tokens"]
    rv.close()


def test_llama8b_backbone_only_decode_equals_forced_full_depth(llama8b, decode_path):
    cfg, c, w = llama8b
    P, S = 256, 4
    L = c["L"]
    outs = []
    for backbone in (False, True):
        rv = river.River(c, w, max_seq=P + S, max_prefill=P)
        toks = synth.prompt(c, 1, P, seed=3, device="cuda")
        pre = rv.prefill(toks, prefill_exit=L)
        if backbone:
            t = rv.decode_backbone_steps(pre["tokens"], S)
        else:
            sched = torch.full((S, 1), L, dtype=torch.int32, device="cuda")
            t = rv.decode_steps(pre["tokens"], sched=sched)
        outs.append((t.cpu().numpy().ravel(), rv.kv_view()[:, :, 0, :, P:P + S].cpu()))
        rv.close()
    assert np.array_equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])


def test_llama8b_64k_context_prefill_and_decode_slices(llama8b, decode_path):
    """The 65536-token configuration at full size, checked on sampled outputs with the GPU's
    own shared cache as the oracle's context (teacher forcing): layer-1 K/V at sampled prompt
    positions (embedding -> norm -> projection -> RoPE), layer-2 K/V at sampled positions far
    into the prompt (one prompt-attention block over up to 65536 positions, then layer 2's
    projection), and whole decode blocks at sampled layers for two decode tokens."""
    _, c, w = llama8b
    cfg = configs.LLAMA_8B_64K
    P, S = cfg["prompt"], 2
    L, Hkv, D = c["L"], c["Hkv"], c["D"]
    rv = river.River(c, w, max_seq=P + S + 2, max_prefill=P)
    assert rv.decode_path() == decode_path
    toks = synth.prompt(c, 1, P, seed=5, device="cuda")
    pre = rv.prefill(toks, prefill_exit=L)
    torch.cuda.synchronize()
    kv = rv.kv_view()
    tk = toks[0].cpu().numpy()
    used = [0, 1, 7, 8, L - 1]  # 0-based layers the checks below run
    orc = O.RiverOracle(c, synth.to_numpy({"embed": w["embed"], "lm_head": w["lm_head"],
                                            "final_norm": w["final_norm"],
                                            "layers": [w["layers"][i] if i in used else None
                                                       for i in range(L)]}),
                        layers=used)
    # layer-1 K/V and layer-2 K/V at sampled prompt positions
    for t in (0, 1, 4097, 40000, P - 1):
        h0 = w["embed"][int(tk[t])].cpu().numpy()
        K1 = kv[0, 0, 0, :, : t + 1].cpu().numpy().copy()
        V1 = kv[0, 1, 0, :, : t + 1].cpu().numpy().copy()
        k1_gpu, v1_gpu = K1[:, t].copy(), V1[:, t].copy()
        h1 = O.block_decode(c, orc.weights_for(0, False), orc.norms(0), h0, t, K1, V1)
        assert rel_err(k1_gpu, K1[:, t]) <= TOL, t
        assert rel_err(v1_gpu, V1[:, t]) <= TOL, t
        lw = orc.weights_for(1, False)
        a = O.rmsnorm(h1, orc.norms(1)["attn_norm"], c["eps"]).astype(np.float64)
        k2 = O.to_f16(lw["wk"] @ a).reshape(Hkv, D)
        v2 = O.to_f16(lw["wv"] @ a).reshape(Hkv, D)
        cs, sn = O.rope_cos_sin(t, D, c["theta"])
        k2 = O.apply_rope(k2, cs, sn)
        assert rel_err(kv[1, 0, 0, :, t].float().cpu().numpy(), k2) <= TOL, t
        assert rel_err(kv[1, 1, 0, :, t].float().cpu().numpy(), v2) <= TOL, t
    # decode blocks at sampled layers
    es = [8, L]  # one early exit and one full-depth token (the config mixes both)
    cur = pre["tokens"]
    for s, e in enumerate(es):
        pos = P + s
        fe = torch.tensor([e], dtype=torch.int32, device="cuda")
        r = rv.decode_step(cur, forced_exit=fe, logits=True)
        assert int(r["exit_layer"][0]) == e
        hs = rv.hidden()[:, 0].cpu().numpy()
        kv = rv.kv_view()
        for l in sorted({1, e, min(e + 1, L), L}):
            Kl = kv[l - 1, 0, 0, :, : pos + 1].cpu().numpy().copy()
            Vl = kv[l - 1, 1, 0, :, : pos + 1].cpu().numpy().copy()
            k_gpu, v_gpu = Kl[:, pos].copy(), Vl[:, pos].copy()
            out = O.block_decode(c, orc.weights_for(l - 1, l > e), orc.norms(l - 1), hs[l - 1], pos, Kl, Vl)
            assert rel_err(hs[l], out) <= TOL, (s, l)
            assert rel_err(k_gpu, Kl[:, pos]) <= TOL, (s, l)
            assert rel_err(v_gpu, Vl[:, pos]) <= TOL, (s, l)
        lg = orc.head_logits(hs[L])
        assert rel_err(r["logits"][0].cpu().numpy(), lg) <= TOL
        assert top1_checked(int(r["tokens"][0]), lg) is not False
        cur = r["tokens"]
    assert rv.positions() == [P + S]
    rv.close()


def test_llama8b_river_export_bit_exact_group128(llama8b):
    """The device quantiser's river copy of one 8B-shape block (group 128; K = 4096 and 14336)
    is bit-exact with the oracle's codes and scales."""
    _, c, w = llama8b
    rv = river.River(c, w, max_seq=16, max_prefill=16)
    layer = 5
    lw = {m: w["layers"][layer][m].cpu().numpy() for m in river.MATS}
    for which, m in enumerate(river.MATS):
        packed, scales = rv.export_river(layer, which)
        q, s = O.quantize_w4(lw[m], c["group"])
        assert np.array_equal(packed.cpu().numpy(), O.pack_nibbles(q)), m
        assert np.array_equal(scales.cpu().numpy().view(np.uint16), s.view(np.uint16)), m
    rv.close()


def _slice_check(c, orc, rv, r, e, pos, layers, tag):
    """Teacher-forced oracle blocks at `layers` on the GPU's own h(l-1) and cache, and the head."""
    L = c["L"]
    hs = rv.hidden()[:, 0].cpu().numpy()
    kv = rv.kv_view()
    for l in layers:
        Kl = kv[l - 1, 0, 0, :, : pos + 1].cpu().numpy().copy()
        Vl = kv[l - 1, 1, 0, :, : pos + 1].cpu().numpy().copy()
        k_gpu, v_gpu = Kl[:, pos].copy(), Vl[:, pos].copy()
        out = O.block_decode(c, orc.weights_for(l - 1, l > e), orc.norms(l - 1), hs[l - 1], pos, Kl, Vl)
        assert rel_err(hs[l], out) <= TOL, (tag, l)
        assert rel_err(k_gpu, Kl[:, pos]) <= TOL, (tag, l)
        assert rel_err(v_gpu, Vl[:, pos]) <= TOL, (tag, l)
    lg = orc.head_logits(hs[L])
    assert rel_err(r["logits"][0].cpu().numpy(), lg) <= TOL, tag
    assert top1_checked(int(r["tokens"][0]), lg) is not False, tag
    return hs


def test_llama8b_chained_launches_match_single_steps_and_oracle(llama8b, decode_path):
    """The bench's launch pattern: 20 forced-schedule steps in one call (persistent path: launches
    of 8, 8 and 4 steps chained on the device) give the same tokens, exit layers and shared cache,
    bit for bit, as 20 single-step calls; steps 9 and 17 of the single-step run are checked
    against oracle blocks at the layers around their exits and the LM head."""
    cfg, c, w = llama8b
    P, S = cfg["prompt"], 20
    L = c["L"]
    sched = torch.from_numpy(synth.schedule(cfg, S, 1, seed=7)).to("cuda")
    es = [int(x) for x in sched[:, 0].cpu()]
    checks = {8: None, 16: None}
    layers = {s: sorted({1, es[s], min(es[s] + 1, L), L}) for s in checks}
    need = sorted({l - 1 for v in layers.values() for l in v})
    orc = O.RiverOracle(c, synth.to_numpy({"embed": w["embed"], "lm_head": w["lm_head"],
                                            "final_norm": w["final_norm"],
                                            "layers": [w["layers"][i] if i in need else None
                                                       for i in range(L)]}), layers=need)
    toks = synth.prompt(c, 1, P, seed=7, device="cuda")
    out = []
    for multi in (True, False):
        rv = river.River(c, w, max_seq=P + S + 2, max_prefill=P)
        assert rv.decode_path() == decode_path
        pre = rv.prefill(toks, prefill_exit=L)
        if multi:
            ex = torch.empty(S, 1, dtype=torch.int32, device="cuda")
            t = rv.decode_steps(pre["tokens"], sched=sched, exit_layer=ex)
            tt, ee = t.cpu().numpy().ravel(), ex.cpu().numpy().ravel()
        else:
            cur, tl, el = pre["tokens"], [], []
            for s in range(S):
                r = rv.decode_step(cur, forced_exit=sched[s], logits=s in checks)
                assert int(r["exit_layer"][0]) == es[s]
                if s in checks:
                    _slice_check(c, orc, rv, r, es[s], P + s, layers[s], ("step", s + 1))
                tl.append(int(r["tokens"][0]))
                el.append(int(r["exit_layer"][0]))
                cur = r["tokens"]
            tt, ee = np.array(tl), np.array(el)
        torch.cuda.synchronize()
        assert rv.device_status() == river.RIVER_OK
        out.append((tt, ee, rv.kv_view()[:, :, 0, :, : P + S].clone()))
        rv.close()
    assert np.array_equal(out[0][1], np.array(es)) and np.array_equal(out[1][1], np.array(es))
    assert np.array_equal(out[0][0], out[1][0])
    assert torch.equal(out[0][2], out[1][2])


def test_llama8b_tau_mode_slices_match_oracle(llama8b, decode_path):
    """Tau mode at the 8B shape: a first step with tau = 2 (never exits) records s(l); tau is then
    set to the median of those similarities so that the next steps exit part-way. Each step's
    similarities are recomputed by the oracle from the GPU's stored residual stream, the exit
    layer must follow the rule wherever |s - tau| > 1e-3, and oracle blocks check the layers
    around the exit."""
    cfg, c, w = llama8b
    P, S = 512, 3
    L = c["L"]
    rv = river.River(c, w, max_seq=P + S + 2, max_prefill=P)
    assert rv.decode_path() == decode_path
    toks = synth.prompt(c, 1, P, seed=9, device="cuda")
    pre = rv.prefill(toks, prefill_exit=L)
    r = rv.decode_step(pre["tokens"], tau=2.0, sim=True)
    assert int(r["exit_layer"][0]) == L
    sv = r["sim"][0].cpu().numpy()
    tau = f32(np.median(sv[~np.isnan(sv)]))
    cur = r["tokens"]
    exits = []
    orc = None
    for s in range(S):
        pos = P + 1 + s
        r = rv.decode_step(cur, tau=tau, logits=True, sim=True)
        e = int(r["exit_layer"][0])
        hs = rv.hidden()[:, 0].cpu().numpy()
        sim = r["sim"][0].cpu().numpy()
        # the GPU's decision against its own stored states: s(l) for l in [entry, e], exit at e
        for l in range(1, L):
            if l <= e and l >= c["entry"]:
                so = O.cosine(hs[l - 1], hs[l])
                assert abs(sim[l - 1] - so) < 1e-4, (s, l, sim[l - 1], so)
                if abs(so - tau) > 1e-3:
                    assert (so > tau) == (l == e), (s, l, so, tau, e)
            else:
                assert np.isnan(sim[l - 1]), (s, l)
        if orc is None:
            need = sorted({0, e - 1, min(e, L - 1), L - 1})
            orc = O.RiverOracle(c, synth.to_numpy({"embed": w["embed"], "lm_head": w["lm_head"],
                                                    "final_norm": w["final_norm"],
                                                    "layers": [w["layers"][i] if i in need else None
                                                               for i in range(L)]}), layers=need)
        lay = sorted(l for l in {1, e, min(e + 1, L), L} if l - 1 in orc.bb)
        _slice_check(c, orc, rv, r, e, pos, lay, ("tau step", s))
        exits.append(e)
        cur = r["tokens"]
    print("tau", tau, "exit layers", exits)
    assert any(e < L for e in exits)
    rv.close()
