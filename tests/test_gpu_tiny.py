"""GPU parity on the tiny decoder (4 layers, d=256): the HIP path through the C ABI against the
CPU oracle, element by element."""

import numpy as np
import pytest
import torch

from oracle import river_oracle as O
from token_level_early_amd import configs, river, synth
from tests._util import TOL, f32, rel_err, top1_checked

pytestmark = pytest.mark.gpu

TINY = configs.model_cfg(configs.TINY)


@pytest.fixture(scope="module")
def tiny():
    w = synth.weights(TINY, seed=0, device="cuda")
    return w, synth.to_numpy(w), O.RiverOracle(TINY, synth.to_numpy(w))


def test_quantizer_export_bit_exact(tiny):
    w, wn, orc = tiny
    rv = river.River(TINY, w, max_seq=16)
    for layer in range(TINY["L"]):
        for which, m in enumerate(river.MATS):
            packed, scales = rv.export_river(layer, which)
            q, s = orc.qcodes[layer][m]
            want_p = O.pack_nibbles(q)
            assert torch.equal(packed.cpu(), torch.from_numpy(want_p)), (layer, m)
            assert np.array_equal(scales.cpu().numpy().view(np.uint16), s.view(np.uint16)), (layer, m)
    rv.close()


def _compare_step(rv, r, o, P, s, tag):
    hs = rv.hidden()[:, 0].float().cpu().numpy()
    assert rel_err(hs, o["hs"][:, 0]) <= TOL, (tag, s, rel_err(hs, o["hs"][:, 0]))
    lg = r["logits"][0].cpu().numpy()
    assert rel_err(lg, o["logits"][0]) <= TOL, (tag, s)
    ok = top1_checked(int(r["tokens"][0]), o["logits"][0])
    assert ok is not False, (tag, s, int(r["tokens"][0]), int(np.argmax(o["logits"][0])))
    assert int(r["exit_layer"][0]) == int(o["exit_layer"][0]), (tag, s)


def _kv_compare(rv, kvo, upto):
    kv = rv.kv_view().float().cpu().numpy()
    for l in range(TINY["L"]):
        for j, ref in ((0, kvo.K), (1, kvo.V)):
            g = kv[l, j, 0, :, :upto]
            assert rel_err(g, ref[l, 0, :, :upto]) <= TOL, (l, j)
    # every slot [0, upto) written on the GPU, nothing beyond
    written = np.abs(kv[:, :, 0]).sum(axis=(1, 2, 4)) > 0  # [L][Tmax]
    assert written[:, :upto].all() and not written[:, upto:].any()


@pytest.mark.parametrize("mode", ["forced2", "tau"])
def test_tiny_prefill_and_decode_match_oracle(tiny, mode, decode_path):
    w, wn, orc = tiny
    cfg = configs.TINY
    P, S = cfg["prompt"], cfg["steps"]
    Tmax = P + S + 8
    rv = river.River(TINY, w, max_seq=Tmax, max_prefill=P)
    assert rv.decode_path() == decode_path
    toks = synth.prompt(TINY, 1, P, seed=0, device="cuda")
    kvo = orc.new_kv(1, Tmax)
    tau = f32(cfg["tau"])
    if mode == "forced2":
        pre = rv.prefill(toks, prefill_exit=TINY["L"], logits=True)
        opre = orc.prefill(kvo, toks.cpu().numpy(), prefill_exit=TINY["L"])
    else:
        pre = rv.prefill(toks, prefill_exit=0, tau=tau, logits=True, min_sim=True)
        ge = pre["seq_exit"].cpu().numpy()
        opre = orc.prefill(kvo, toks.cpu().numpy(), tau=tau, gpu_seq_exit=ge)
        assert int(ge[0]) == int(opre["seq_exit"][0])
    torch.cuda.synchronize()
    assert rel_err(pre["logits"][0].cpu().numpy(), opre["logits"][0]) <= TOL
    assert top1_checked(int(pre["tokens"][0]), opre["logits"][0]) is not False
    _kv_compare(rv, kvo, P)
    cur = pre["tokens"]
    exits = []
    for s in range(S):
        if mode == "forced2":
            fe = torch.tensor([cfg["forced_exit"]], dtype=torch.int32, device="cuda")
            r = rv.decode_step(cur, forced_exit=fe, logits=True)
            o = orc.decode_step(kvo, cur.cpu().numpy(), forced_exit=[cfg["forced_exit"]])
        else:
            r = rv.decode_step(cur, tau=tau, logits=True, sim=True)
            ge = r["exit_layer"].cpu().numpy()
            o = orc.decode_step(kvo, cur.cpu().numpy(), tau=tau, gpu_exit=ge)
            sim = r["sim"][0].cpu().numpy()
            osim = o["sim"][0]
            assert np.array_equal(np.isnan(sim), np.isnan(osim)), s
            fin = ~np.isnan(osim)
            assert np.allclose(sim[fin], osim[fin], atol=2e-3), s
        _compare_step(rv, r, o, P, s, mode)
        exits.append(int(r["exit_layer"][0]))
        cur = r["tokens"]
    _kv_compare(rv, kvo, P + S)
    assert rv.positions() == [P + S]
    assert rv.device_status() == river.RIVER_OK
    if mode == "forced2":
        assert set(exits) == {2}
    rv.close()


def test_tau_extremes(tiny, decode_path):
    w, wn, orc = tiny
    rv = river.River(TINY, w, max_seq=64)
    toks = synth.prompt(TINY, 1, 8, seed=1, device="cuda")
    pre = rv.prefill(toks, prefill_exit=TINY["L"])
    cur = pre["tokens"]
    r = rv.decode_step(cur, tau=1.5)
    assert int(r["exit_layer"][0]) == TINY["L"]
    r = rv.decode_step(r["tokens"], tau=-1.5)
    assert int(r["exit_layer"][0]) == TINY["entry"]
    rv.close()


def test_forced_exit_out_of_range_flags_device_error(tiny):
    w, wn, orc = tiny
    rv = river.River(TINY, w, max_seq=64)
    toks = synth.prompt(TINY, 1, 8, seed=1, device="cuda")
    pre = rv.prefill(toks, prefill_exit=TINY["L"])
    fe = torch.tensor([TINY["L"] + 5], dtype=torch.int32, device="cuda")
    r = rv.decode_step(pre["tokens"], forced_exit=fe)
    assert rv.device_status() == river.RIVER_EDEVICE
    assert int(r["exit_layer"][0]) == TINY["L"]  # treated as no exit
    assert rv.device_status() == river.RIVER_OK  # cleared
    rv.close()


def test_position_overflow_is_rejected_on_host(tiny):
    w, wn, orc = tiny
    rv = river.River(TINY, w, max_seq=10, max_prefill=10)
    toks = synth.prompt(TINY, 1, 10, seed=1, device="cuda")
    pre = rv.prefill(toks, prefill_exit=TINY["L"])
    with pytest.raises(river.RiverError) as e:
        rv.decode_step(pre["tokens"], tau=0.5)
    assert e.value.code == river.RIVER_ERANGE
    rv.close()


def test_multi_step_matches_single_steps(tiny, decode_path):
    w, wn, orc = tiny
    S = 6
    sched = torch.tensor([[1], [2], [3], [4], [2], [1]], dtype=torch.int32, device="cuda")
    outs = []
    for multi in (False, True):
        rv = river.River(TINY, w, max_seq=64)
        toks = synth.prompt(TINY, 1, 16, seed=2, device="cuda")
        pre = rv.prefill(toks, prefill_exit=TINY["L"])
        if multi:
            ex = torch.empty(S, 1, dtype=torch.int32, device="cuda")
            t = rv.decode_steps(pre["tokens"], sched=sched, exit_layer=ex)
            outs.append((t.cpu().numpy().ravel(), ex.cpu().numpy().ravel(), rv.kv_view().cpu()))
        else:
            cur, tt, ee = pre["tokens"], [], []
            for s in range(S):
                r = rv.decode_step(cur, forced_exit=sched[s])
                tt.append(int(r["tokens"][0]))
                ee.append(int(r["exit_layer"][0]))
                cur = r["tokens"]
            outs.append((np.array(tt), np.array(ee), rv.kv_view().cpu()))
        rv.close()
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1]) and list(outs[0][1]) == [1, 2, 3, 4, 2, 1]
    assert torch.equal(outs[0][2], outs[1][2])  # deterministic, bit-identical cache


def _run_path(w, persist, tau=None, sched=None, P=16, S=6):
    import os
    old = os.environ.get("RIVER_PERSIST")
    os.environ["RIVER_PERSIST"] = "1" if persist else "0"
    try:
        rv = river.River(TINY, w, max_seq=P + S + 2, max_prefill=P)
    finally:
        if old is None:
            del os.environ["RIVER_PERSIST"]
        else:
            os.environ["RIVER_PERSIST"] = old
    toks = synth.prompt(TINY, 1, P, seed=4, device="cuda")
    pre = rv.prefill(toks, prefill_exit=TINY["L"])
    ex = torch.empty(S, 1, dtype=torch.int32, device="cuda")
    sim = torch.empty(S, 1, TINY["L"], dtype=torch.float32, device="cuda")
    if sched is not None:
        t = rv.decode_steps(pre["tokens"], sched=sched, exit_layer=ex)
    else:
        t = rv.decode_steps(pre["tokens"], S=S, tau=tau, exit_layer=ex, sim=sim)
    out = (t.cpu().numpy().ravel(), ex.cpu().numpy().ravel(), sim.cpu().numpy(),
           rv.hidden().float().cpu().numpy(), rv.kv_view().float().cpu().numpy(), rv.positions())
    assert rv.device_status() == river.RIVER_OK
    rv.close()
    return out


@pytest.mark.parametrize("mode", ["forced", "tau"])
def test_persistent_kernel_matches_per_op_kernels(tiny, mode):
    w, wn, orc = tiny
    S = 6
    sched = torch.tensor([[1], [3], [2], [4], [2], [1]], dtype=torch.int32, device="cuda")
    kw = {"sched": sched} if mode == "forced" else {"tau": f32(0.2)}
    a = _run_path(w, True, S=S, **kw)
    b = _run_path(w, False, S=S, **kw)
    assert a[5] == b[5]
    assert np.array_equal(a[1], b[1])  # exit layers
    assert rel_err(a[3], b[3]) <= TOL  # last step's residual stream
    assert rel_err(a[4], b[4]) <= TOL  # whole shared cache
    agree = (a[0] == b[0]).mean()
    assert agree >= 5 / 6, (a[0], b[0])
    if mode == "tau":
        fin = ~np.isnan(b[2])
        assert np.array_equal(np.isnan(a[2]), np.isnan(b[2]))
        assert np.allclose(a[2][fin], b[2][fin], atol=2e-3)


def test_persistent_tags_wrap_and_long_context_switch(tiny):
    """The persistent kernel's 16-bit activation tags wrap after 65535 uses (13107 steps of the
    4-layer decoder), and launches that reach position 8192 switch to the long-context kernel
    variant. Decoding 13200 steps across both raises no device error (a stale tag matching, or
    a wait that never ends, would abort the launch and set the error word) and is deterministic:
    two contexts decoding the same prompt produce the same tokens and residual stream."""
    import os
    w, wn, orc = tiny
    P, S = 16, 13200
    old = os.environ.get("RIVER_PERSIST")
    os.environ["RIVER_PERSIST"] = "1"
    outs = []
    try:
        for _ in range(2):
            rv = river.River(TINY, w, max_seq=P + S + 2, max_prefill=P)
            assert rv.decode_path() == "persistent"
            toks = synth.prompt(TINY, 1, P, seed=5, device="cuda")
            pre = rv.prefill(toks, prefill_exit=TINY["L"])
            sched = torch.full((S, 1), 2, dtype=torch.int32, device="cuda")
            t = rv.decode_steps(pre["tokens"], sched=sched)
            torch.cuda.synchronize()
            assert rv.device_status() == river.RIVER_OK
            assert rv.positions() == [P + S]
            outs.append((t.cpu().numpy().ravel(), rv.hidden().float().cpu().numpy()))
            rv.close()
    finally:
        if old is None:
            del os.environ["RIVER_PERSIST"]
        else:
            os.environ["RIVER_PERSIST"] = old
    toks0, hs0 = outs[0]
    assert ((toks0 >= 0) & (toks0 < TINY["V"])).all()
    assert np.array_equal(toks0, outs[1][0])
    assert np.array_equal(hs0, outs[1][1])


def test_tiny_forced_zero_all_river_matches_oracle(tiny, decode_path):
    """Forced exit 0 runs every block on the river (the all-int4 "Full Quantization" comparator,
    paperlayer summary §5). A schedule mixing 0 with ordinary exits, on both decode paths,
    against the oracle step by step (teacher-forced with the GPU's tokens); the multi-step call
    gives the same exits and tokens as the single steps."""
    w, wn, orc = tiny
    L, P = TINY["L"], 16
    sched = [0, 0, 3, 0, 1, L, 0]
    S = len(sched)
    rv = river.River(TINY, w, max_seq=P + S + 4, max_prefill=P)
    assert rv.decode_path() == decode_path
    toks = synth.prompt(TINY, 1, P, seed=2, device="cuda")
    kvo = orc.new_kv(1, P + S + 4)
    pre = rv.prefill(toks, prefill_exit=L)
    orc.prefill(kvo, toks.cpu().numpy(), prefill_exit=L)
    cur = pre["tokens"]
    got = []
    for s, e in enumerate(sched):
        fe = torch.tensor([e], dtype=torch.int32, device="cuda")
        r = rv.decode_step(cur, forced_exit=fe, logits=True)
        o = orc.decode_step(kvo, cur.cpu().numpy(), forced_exit=[e])
        assert int(r["exit_layer"][0]) == e == int(o["exit_layer"][0]), s
        _compare_step(rv, r, o, P, s, "forced0")
        cur = r["tokens"]
        got.append(int(cur[0]))
    _kv_compare(rv, kvo, P + S)
    assert rv.device_status() == river.RIVER_OK
    rv.close()

    rv = river.River(TINY, w, max_seq=P + S + 4, max_prefill=P)
    pre = rv.prefill(toks, prefill_exit=L)
    ex = torch.empty(S, 1, dtype=torch.int32, device="cuda")
    sch = torch.tensor(sched, dtype=torch.int32, device="cuda").view(S, 1)
    t = rv.decode_steps(pre["tokens"], sched=sch, exit_layer=ex)
    assert ex.cpu().numpy().ravel().tolist() == sched
    assert t.cpu().numpy().ravel().tolist() == got
    assert rv.device_status() == river.RIVER_OK
    rv.close()


def test_prefill_after_decode_reuses_context(tiny, decode_path):
    """A context that decoded (an odd number of steps, which leaves the persistent kernel's
    last argmax key in slot 0) and is then prefilled with another prompt gives exactly what a
    fresh context gives for that prompt, and the oracle's answer."""
    w, wn, orc = tiny
    L, P = TINY["L"], 12
    t1 = synth.prompt(TINY, 1, P, seed=21, device="cuda")
    t2 = synth.prompt(TINY, 1, P, seed=22, device="cuda")
    rv = river.River(TINY, w, max_seq=P + 8, max_prefill=P)
    assert rv.decode_path() == decode_path
    pre = rv.prefill(t1, prefill_exit=L)
    r = rv.decode_step(pre["tokens"], forced_exit=torch.tensor([2], dtype=torch.int32, device="cuda"))
    rv.decode_steps(r["tokens"], sched=torch.tensor([[1], [3], [L]], dtype=torch.int32, device="cuda"))
    again = rv.prefill(t2, prefill_exit=L, logits=True)
    torch.cuda.synchronize()
    assert rv.positions() == [P]
    fresh = river.River(TINY, w, max_seq=P + 8, max_prefill=P)
    ref = fresh.prefill(t2, prefill_exit=L, logits=True)
    torch.cuda.synchronize()
    assert int(again["tokens"][0]) == int(ref["tokens"][0])
    assert torch.equal(again["logits"], ref["logits"])
    kvo = orc.new_kv(1, P + 8)
    o = orc.prefill(kvo, t2.cpu().numpy(), prefill_exit=L)
    assert rel_err(again["logits"][0].cpu().numpy(), o["logits"][0]) <= TOL
    assert top1_checked(int(again["tokens"][0]), o["logits"][0]) is not False
    # and decoding continues from position P as on the fresh context
    a = rv.decode_step(again["tokens"], forced_exit=torch.tensor([1], dtype=torch.int32, device="cuda"))
    b = fresh.decode_step(ref["tokens"], forced_exit=torch.tensor([1], dtype=torch.int32, device="cuda"))
    assert int(a["tokens"][0]) == int(b["tokens"][0])
    assert torch.equal(rv.kv_view()[:, :, 0, :, : P + 1], fresh.kv_view()[:, :, 0, :, : P + 1])
    rv.close()
    fresh.close()


@pytest.mark.parametrize("mode", ["forced", "tau"])
def test_chained_launches_equal_single_steps(tiny, mode, decode_path):
    """S = 20 decode steps in one call -- on the persistent path three chained launches of at
    most 8 steps, each starting from the previous launch's last token and tag counter -- give
    bit for bit the tokens, exit layers, similarities and shared cache of 20 single-step calls;
    the last step's residual stream matches the oracle teacher-forced with the GPU's tokens."""
    w, wn, orc = tiny
    L, P, S = TINY["L"], 16, 20
    rng = np.random.default_rng(17)
    sched_np = rng.integers(0, L + 1, size=(S, 1)).astype(np.int32)
    tau = f32(0.3)
    toks = synth.prompt(TINY, 1, P, seed=23, device="cuda")
    runs = []
    for multi in (True, False):
        rv = river.River(TINY, w, max_seq=P + S + 2, max_prefill=P)
        assert rv.decode_path() == decode_path
        pre = rv.prefill(toks, prefill_exit=L)
        if multi:
            ex = torch.empty(S, 1, dtype=torch.int32, device="cuda")
            sim = torch.empty(S, 1, L, dtype=torch.float32, device="cuda")
            if mode == "forced":
                t = rv.decode_steps(pre["tokens"], sched=torch.from_numpy(sched_np).cuda(), exit_layer=ex, sim=sim)
            else:
                t = rv.decode_steps(pre["tokens"], S=S, tau=tau, exit_layer=ex, sim=sim)
            tt, ee, ss = t.cpu().numpy().ravel(), ex.cpu().numpy().ravel(), sim.cpu().numpy()[:, 0]
        else:
            cur, tl, el, sl = pre["tokens"], [], [], []
            for s in range(S):
                if mode == "forced":
                    r = rv.decode_step(cur, forced_exit=torch.from_numpy(sched_np[s]).cuda())
                else:
                    r = rv.decode_step(cur, tau=tau)
                tl.append(int(r["tokens"][0]))
                el.append(int(r["exit_layer"][0]))
                sl.append(r["sim"][0].cpu().numpy())
                cur = r["tokens"]
            tt, ee, ss = np.array(tl), np.array(el), np.stack(sl)
        torch.cuda.synchronize()
        assert rv.device_status() == river.RIVER_OK
        runs.append((tt, ee, ss, rv.kv_view().cpu(), rv.hidden().cpu(), rv.positions(),
                     int(pre["tokens"][0])))
        rv.close()
    (ta, ea, sa, ka, ha, pa, first), (tb, eb, sb, kb, hb, pb, _) = runs
    assert pa == pb == [P + S]
    assert np.array_equal(ta, tb) and np.array_equal(ea, eb)
    assert np.array_equal(np.isnan(sa), np.isnan(sb)) and np.array_equal(sa[~np.isnan(sa)], sb[~np.isnan(sb)])
    assert torch.equal(ka, kb) and torch.equal(ha, hb)
    if mode == "forced":
        assert np.array_equal(ea, sched_np.ravel())
    # oracle over the same 20 steps, teacher-forced with the GPU's tokens (and its decisions
    # inside the tau margin)
    kvo = orc.new_kv(1, P + S + 2)
    orc.prefill(kvo, toks.cpu().numpy(), prefill_exit=L)
    cur = first
    for s in range(S):
        if mode == "forced":
            o = orc.decode_step(kvo, [cur], forced_exit=[int(sched_np[s, 0])])
        else:
            o = orc.decode_step(kvo, [cur], tau=tau, gpu_exit=[int(ea[s])])
        assert int(o["exit_layer"][0]) == int(ea[s]), s
        cur = int(ta[s])
    assert rel_err(ha[:, 0].float().numpy(), o["hs"][:, 0]) <= TOL
    assert rel_err(ka.float().numpy()[:, :, 0], np.stack([kvo.K[:, 0], kvo.V[:, 0]], axis=1)) <= TOL


@pytest.mark.parametrize("batch", [1, 3])
def test_chunked_prefill_matches_whole_prefill_and_oracle(tiny, batch):
    """Prefill in chunks of 24 positions (64-token prompt: chunks 24, 24 and a ragged 16) gives
    bit for bit the shared cache, exit layers, similarities and logits of a single-chunk prefill
    (every output element is the same computation), and matches the oracle, in tau mode where
    the sequence-level exit needs the similarities of every chunk's tokens."""
    w, wn, orc = tiny
    P = 64
    tau = f32(0.95)
    toks = synth.prompt(TINY, batch, P, seed=31, device="cuda")
    runs = []
    for chunk in (24, 0):
        c = dict(TINY, prefill_chunk=chunk)
        rv = river.River(c, w, max_seq=P + 2, max_prefill=P, batch=batch)
        pre = rv.prefill(toks, prefill_exit=0, tau=tau, logits=True, min_sim=True)
        torch.cuda.synchronize()
        runs.append({k: (v.cpu() if v is not None else None) for k, v in pre.items()})
        runs[-1]["kv"] = rv.kv_view().cpu()
        rv.close()
    a, b = runs
    for k in ("tokens", "logits", "seq_exit", "kv"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(torch.isnan(a["min_sim"]), torch.isnan(b["min_sim"]))
    kvo = orc.new_kv(batch, P + 2)
    o = orc.prefill(kvo, toks.cpu().numpy(), tau=tau, gpu_seq_exit=a["seq_exit"].numpy())
    assert np.array_equal(a["seq_exit"].numpy(), o["seq_exit"])
    for r in range(batch):
        assert rel_err(a["logits"][r].numpy(), o["logits"][r]) <= TOL
        assert top1_checked(int(a["tokens"][r]), o["logits"][r]) is not False
        fin = ~np.isnan(o["min_sim"][r])
        assert np.allclose(a["min_sim"][r].numpy()[fin], o["min_sim"][r][fin], atol=2e-3)
    kv = a["kv"].float().numpy()
    for l in range(TINY["L"]):
        assert rel_err(kv[l, 0, :, :, :P], kvo.K[l, :, :, :P]) <= TOL, l
        assert rel_err(kv[l, 1, :, :, :P], kvo.V[l, :, :, :P]) <= TOL, l
