"""river_decode_steps_static -- the decode entry point for callers that cannot allocate device
memory, with the persistent kernel's exchange buffers in the library's fixed device array --
against river_decode_steps on identical contexts: two calls in a row (the second with fewer
steps) give bit for bit the same tokens, exit layers, similarities, residual stream, shared
cache and positions. Sizes beyond the array and contexts off the persistent kernel are rejected
with an error before any device work."""

import os

import numpy as np
import pytest
import torch

from token_level_early_amd import configs, river, synth
from tests._util import f32

pytestmark = pytest.mark.gpu

TINY = configs.model_cfg(configs.TINY)


def _persistent_ctx(c, w, **kw):
    old = os.environ.get("RIVER_PERSIST")
    os.environ["RIVER_PERSIST"] = "1"
    try:
        return river.River(c, w, **kw)
    finally:
        if old is None:
            del os.environ["RIVER_PERSIST"]
        else:
            os.environ["RIVER_PERSIST"] = old


def _run(c, w, P, calls, static, mode, tau, seed):
    rv = _persistent_ctx(c, w, max_seq=P + sum(n for n, _ in calls) + 2, max_prefill=P)
    assert rv.decode_path() == "persistent"
    toks = synth.prompt(c, 1, P, seed=seed, device="cuda")
    cur = rv.prefill(toks, prefill_exit=c["L"])["tokens"]
    outs = []
    for n, sched in calls:
        ex = torch.empty(n, 1, dtype=torch.int32, device="cuda")
        sim = torch.empty(n, 1, c["L"], dtype=torch.float32, device="cuda")
        fn = rv.decode_steps_static if static else rv.decode_steps
        if mode == "forced":
            t = fn(cur, sched=sched, exit_layer=ex, sim=sim)
        else:
            t = fn(cur, S=n, tau=tau, exit_layer=ex, sim=sim)
        torch.cuda.synchronize()
        assert rv.device_status() == river.RIVER_OK
        outs.append((t.cpu().numpy(), ex.cpu().numpy(), sim.cpu().numpy(), rv.hidden().cpu(),
                     rv.positions()))
        cur = t[-1].clone()
    kv = rv.kv_view().cpu()
    rv.close()
    return outs, kv


def _same(a, b):
    (oa, ka), (ob, kb) = a, b
    assert torch.equal(ka, kb)
    for x, y in zip(oa, ob):
        assert np.array_equal(x[0], y[0]) and np.array_equal(x[1], y[1])
        assert np.array_equal(np.isnan(x[2]), np.isnan(y[2]))
        assert np.array_equal(x[2][~np.isnan(x[2])], y[2][~np.isnan(y[2])])
        assert torch.equal(x[3], y[3]) and x[4] == y[4]


@pytest.mark.parametrize("mode", ["forced", "tau"])
def test_static_scratch_decode_equals_decode_steps_tiny(mode):
    w = synth.weights(TINY, seed=0, device="cuda")
    rng = np.random.default_rng(31)
    calls = [(n, torch.from_numpy(rng.integers(0, TINY["L"] + 1, size=(n, 1)).astype(np.int32)).cuda())
             for n in (13, 5)]  # two launches, then one shorter launch
    ref = _run(TINY, w, 16, calls, False, mode, f32(0.3), 41)
    got = _run(TINY, w, 16, calls, True, mode, f32(0.3), 41)
    _same(ref, got)


def test_static_scratch_decode_equals_decode_steps_llama8b():
    cfg = configs.LLAMA_8B
    c = configs.model_cfg(cfg)
    w = synth.weights(c, seed=0, device="cuda")
    sched = torch.from_numpy(synth.schedule(cfg, 14, 1, seed=3)).cuda()
    calls = [(10, sched[:10].contiguous()), (4, sched[10:].contiguous())]
    ref = _run(c, w, 256, calls, False, "forced", 0.0, 43)
    got = _run(c, w, 256, calls, True, "forced", 0.0, 43)
    _same(ref, got)


def test_static_scratch_rejects_oversized_and_non_persistent_contexts():
    # 2048 tiny layers (all borrowing one layer's weights): the exchange buffers (h and h_mid of
    # every layer) pass the array's 4 MiB
    c = dict(TINY, L=2048)
    w1 = synth.weights(TINY, seed=0, device="cuda")
    w = {"embed": w1["embed"], "lm_head": w1["lm_head"], "final_norm": w1["final_norm"],
         "layers": [w1["layers"][0]] * c["L"]}
    rv = _persistent_ctx(c, w, max_seq=8, max_prefill=4)
    assert rv.decode_path() == "persistent"
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(river.RiverError) as e:
        rv.decode_steps_static(tok, S=1, tau=0.5)
    assert e.value.code == river.RIVER_ENOMEM and "static scratch holds" in str(e.value)
    assert rv.positions() == [0]
    rv.close()
    rb = river.River(TINY, w1, max_seq=8, max_prefill=4, batch=2)
    with pytest.raises(river.RiverError) as e:
        rb.decode_steps_static(torch.zeros(2, dtype=torch.int32, device="cuda"), S=1, tau=0.5)
    assert e.value.code == river.RIVER_EINVAL
    rb.close()
