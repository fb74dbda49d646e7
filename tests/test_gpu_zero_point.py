"""GPU parity of the zero-point river format (scale and integer zero point per group: the
storage of the pages' other backends, paperlayer.ai summary of arXiv 2604.18396v3, appendix A.1)
against the oracle with the same format: the device quantiser's export bit for bit (tiny with
its ragged 48-element group, and one 8B-shape block at group 128), prefill and decode on the
persistent and per-op kernels (forced schedules with 0 and L, tau mode), batch 4 on the batched
kernels, and sampled 8B-shape decode blocks."""

import numpy as np
import pytest
import torch

from oracle import river_oracle as O
from token_level_early_amd import configs, river, synth
from tests._util import TOL, f32, rel_err, top1_checked

pytestmark = pytest.mark.gpu

TZ = configs.model_cfg(configs.TINY_ZP)


@pytest.fixture(scope="module")
def tiny():
    w = synth.weights(TZ, seed=0, device="cuda")
    return w, O.RiverOracle(TZ, synth.to_numpy(w))


def test_zp_export_bit_exact_tiny(tiny):
    w, orc = tiny
    rv = river.River(TZ, w, max_seq=16)
    for layer in range(TZ["L"]):
        for which, m in enumerate(river.MATS):
            packed, scales, zeros = rv.export_river(layer, which)
            q, s, z = orc.qcodes[layer][m]
            assert np.array_equal(packed.cpu().numpy(), O.pack_codes(q)), (layer, m)
            assert np.array_equal(scales.cpu().numpy().view(np.uint16), s.view(np.uint16)), (layer, m)
            assert np.array_equal(zeros.cpu().numpy(), z), (layer, m)
    rv.close()


def test_zp_export_bit_exact_llama8b_block():
    c = configs.model_cfg(configs.LLAMA_8B_ZP)
    w = synth.weights(c, seed=0, device="cuda", layers=[0, 3])
    layers = [w["layers"][i] if i in (0, 3) else w["layers"][0] for i in range(c["L"])]
    rv = river.River(c, dict(w, layers=layers), max_seq=16, max_prefill=16)
    for which, m in enumerate(river.MATS):
        packed, scales, zeros = rv.export_river(3, which)
        q, s, z = O.quantize_w4_zp(w["layers"][3][m].cpu().numpy(), c["group"])
        assert np.array_equal(packed.cpu().numpy(), O.pack_codes(q)), m
        assert np.array_equal(scales.cpu().numpy().view(np.uint16), s.view(np.uint16)), m
        assert np.array_equal(zeros.cpu().numpy(), z), m
    rv.close()


@pytest.mark.parametrize("mode", ["forced", "tau"])
def test_zp_tiny_prefill_and_decode_match_oracle(tiny, mode, decode_path):
    w, orc = tiny
    L, P, S = TZ["L"], 32, 12
    Tmax = P + S + 2
    rv = river.River(TZ, w, max_seq=Tmax, max_prefill=P)
    assert rv.decode_path() == decode_path
    toks = synth.prompt(TZ, 1, P, seed=5, device="cuda")
    kvo = orc.new_kv(1, Tmax)
    if mode == "forced":  # prefill on the river after layer 2
        pre = rv.prefill(toks, prefill_exit=2, logits=True)
        opre = orc.prefill(kvo, toks.cpu().numpy(), prefill_exit=2)
    else:
        tau = f32(0.95)
        pre = rv.prefill(toks, prefill_exit=0, tau=tau, logits=True)
        ge = pre["seq_exit"].cpu().numpy()
        opre = orc.prefill(kvo, toks.cpu().numpy(), tau=tau, gpu_seq_exit=ge)
        assert int(ge[0]) == int(opre["seq_exit"][0])
    assert rel_err(pre["logits"][0].cpu().numpy(), opre["logits"][0]) <= TOL
    assert top1_checked(int(pre["tokens"][0]), opre["logits"][0]) is not False
    sched = [0, L, 1, 2, 3, 0, 2, 1, L, 3, 0, 1]
    cur = pre["tokens"]
    for s in range(S):
        if mode == "forced":
            fe = torch.tensor([sched[s]], dtype=torch.int32, device="cuda")
            r = rv.decode_step(cur, forced_exit=fe, logits=True)
            o = orc.decode_step(kvo, cur.cpu().numpy(), forced_exit=[sched[s]])
        else:
            r = rv.decode_step(cur, tau=f32(0.3), logits=True)
            o = orc.decode_step(kvo, cur.cpu().numpy(), tau=f32(0.3), gpu_exit=r["exit_layer"].cpu().numpy())
        assert int(r["exit_layer"][0]) == int(o["exit_layer"][0]), s
        hs = rv.hidden()[:, 0].float().cpu().numpy()
        assert rel_err(hs, o["hs"][:, 0]) <= TOL, (s, rel_err(hs, o["hs"][:, 0]))
        assert rel_err(r["logits"][0].cpu().numpy(), o["logits"][0]) <= TOL, s
        assert top1_checked(int(r["tokens"][0]), o["logits"][0]) is not False, s
        cur = r["tokens"]
    kv = rv.kv_view().float().cpu().numpy()
    for l in range(L):
        assert rel_err(kv[l, 0, 0, :, :P + S], kvo.K[l, 0, :, :P + S]) <= TOL, l
        assert rel_err(kv[l, 1, 0, :, :P + S], kvo.V[l, 0, :, :P + S]) <= TOL, l
    assert rv.device_status() == river.RIVER_OK
    rv.close()


def test_zp_tiny_batch4_matches_oracle(tiny):
    w, orc = tiny
    B, P, S = 4, 24, 6
    L = TZ["L"]
    rv = river.River(TZ, w, max_seq=P + S + 2, max_prefill=P, batch=B)
    toks = synth.prompt(TZ, B, P, seed=8, device="cuda")
    kvo = orc.new_kv(B, P + S + 2)
    pre = rv.prefill(toks, prefill_exit=L)
    orc.prefill(kvo, toks.cpu().numpy(), prefill_exit=L)
    rng = np.random.default_rng(9)
    cur = pre["tokens"]
    for s in range(S):
        fe = rng.integers(0, L + 1, size=B).astype(np.int32)
        r = rv.decode_step(cur, forced_exit=torch.from_numpy(fe).cuda(), logits=True)
        o = orc.decode_step(kvo, cur.cpu().numpy(), forced_exit=list(fe))
        hs = rv.hidden().float().cpu().numpy()
        for b in range(B):
            assert rel_err(hs[:, b], o["hs"][:, b]) <= TOL, (s, b)
            assert rel_err(r["logits"][b].cpu().numpy(), o["logits"][b]) <= TOL, (s, b)
            assert top1_checked(int(r["tokens"][b]), o["logits"][b]) is not False, (s, b)
        cur = r["tokens"]
    rv.close()


def test_zp_llama8b_decode_slices_match_oracle(decode_path):
    cfg = configs.LLAMA_8B_ZP
    c = configs.model_cfg(cfg)
    P, S = 256, 3
    L = c["L"]
    w = synth.weights(c, seed=0, device="cuda")
    rv = river.River(c, w, max_seq=P + S + 2, max_prefill=P)
    assert rv.decode_path() == decode_path
    toks = synth.prompt(c, 1, P, seed=6, device="cuda")
    es = [0, 9, 20]
    need = sorted({0, 8, 9, 19, 20, L - 1})
    orc = O.RiverOracle(c, synth.to_numpy({"embed": w["embed"], "lm_head": w["lm_head"],
                                            "final_norm": w["final_norm"],
                                            "layers": [w["layers"][i] if i in need else None
                                                       for i in range(L)]}), layers=need)
    cur = rv.prefill(toks, prefill_exit=L)["tokens"]
    for s, e in enumerate(es):
        pos = P + s
        r = rv.decode_step(cur, forced_exit=torch.tensor([e], dtype=torch.int32, device="cuda"), logits=True)
        assert int(r["exit_layer"][0]) == e
        hs = rv.hidden()[:, 0].cpu().numpy()
        kv = rv.kv_view()
        for l in sorted({1, max(e, 1), min(e + 1, L), L}):
            if l - 1 not in need:
                continue
            Kl = kv[l - 1, 0, 0, :, : pos + 1].cpu().numpy().copy()
            Vl = kv[l - 1, 1, 0, :, : pos + 1].cpu().numpy().copy()
            k_gpu, v_gpu = Kl[:, pos].copy(), Vl[:, pos].copy()
            out = O.block_decode(c, orc.weights_for(l - 1, l > e), orc.norms(l - 1), hs[l - 1], pos, Kl, Vl)
            assert rel_err(hs[l], out) <= TOL, (s, l)
            assert rel_err(k_gpu, Kl[:, pos]) <= TOL and rel_err(v_gpu, Vl[:, pos]) <= TOL, (s, l)
        lg = orc.head_logits(hs[L])
        assert rel_err(r["logits"][0].cpu().numpy(), lg) <= TOL
        assert top1_checked(int(r["tokens"][0]), lg) is not False
        cur = r["tokens"]
    assert rv.device_status() == river.RIVER_OK
    rv.close()
