"""Measures the end-to-end noise floor behind the end-to-end tolerance of the GPU parity tests
(no GPU). The same oracle decoder (Llama-3.2-1B shape: 16 blocks, N(0, 0.02) weights) is run
twice: once as written (every linear map accumulated in fp64) and once with every linear map
accumulated in fp32 (numpy float32 products and BLAS summation order) -- the same algorithm
with the same fp16 storage points, differing only in the accumulation precision an fp32 GPU
kernel has. The fp16 roundings that flip between the two compound through the blocks: the
logits differ by about 1.0-1.2e-2 of their rms, the final hidden state by about 0.8-0.95e-2
(measured on four positions). So no fp32-
accumulating implementation can be held to 1e-2 end to end against the fp64 oracle; the GPU
tests hold every block and the head to 1e-2 on identical inputs (the GPU's own h(l-1) and
cache), and the end-to-end states to TOL_E2E = 3e-2 (at least twice the floor measured here)
plus identical top-1 tokens outside near-ties."""

import numpy as np
import pytest

from oracle import river_oracle as O
from token_level_early_amd import configs, synth
from tests._util import TOL, TOL_E2E, rel_err

pytestmark = pytest.mark.slow


def test_fp32_accumulation_floor_exceeds_the_per_block_bound_end_to_end(monkeypatch):
    c = configs.model_cfg(configs.LLAMA_1B)
    L = c["L"]
    w = synth.to_numpy(synth.weights(c, seed=0, device="cpu"))
    mats = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")
    norms = [{"attn_norm": w["layers"][i]["attn_norm"], "mlp_norm": w["layers"][i]["mlp_norm"]}
             for i in range(L)]
    head = w["embed"].astype(np.float64)  # tied
    lin64 = O._lin

    def lin32(W, x16):
        return (np.asarray(x16).astype(np.float32) @ np.asarray(W, np.float32).T).astype(np.float64)

    def run(tokens, dtype, lin):
        W = [{m: w["layers"][i][m].astype(dtype) for m in mats} for i in range(L)]
        monkeypatch.setattr(O, "_lin", lin)
        K = np.zeros((L, c["Hkv"], len(tokens), c["D"]), np.float16)
        V = np.zeros_like(K)
        out = []
        for pos, tok in enumerate(tokens):
            h = w["embed"][tok].copy()
            for l in range(L):
                h = O.block_decode(c, W[l], norms[l], h, pos, K[l], V[l])
            x = O.rmsnorm(h, w["final_norm"], c["eps"]).astype(np.float64)
            out.append((h, x @ head.T))
        monkeypatch.setattr(O, "_lin", lin64)
        return out

    toks = synth.prompt(c, 1, 4, seed=0).numpy()[0]
    ref = run(toks, np.float64, lin64)
    f32 = run(toks, np.float32, lin32)
    lg = [rel_err(b[1], a[1]) for a, b in zip(ref, f32)]
    hs = [rel_err(b[0], a[0]) for a, b in zip(ref, f32)]
    print("fp32-accumulation floor, logits:", [round(x, 5) for x in lg], "h(L):", [round(x, 5) for x in hs])
    assert max(lg) > TOL and min(lg) > 0.8 * TOL, lg  # the logits: above the per-block bound
    assert min(hs) > 0.5 * TOL, hs                     # the final state: the same order
    assert TOL_E2E >= 2 * max(lg + hs), (lg, hs)       # the end-to-end bound leaves 2x headroom
