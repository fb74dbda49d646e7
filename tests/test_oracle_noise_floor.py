"""Measures the end-to-end noise floor that justifies the end-to-end tolerance of the GPU
parity tests (no GPU): in the 16-block Llama-3.2-1B-shaped decoder with N(0, 0.02) weights,
a one-ulp change of a few fp16 values of h(1) -- the kind of rounding difference an fp32
accumulating kernel has against the fp64 oracle -- moves the final logits by a large fraction
of the 1e-2 per-block bound. Per-block agreement is therefore checked at 1e-2 and end-to-end
agreement at 3e-2 with exact top-1 tokens outside near-ties."""

import numpy as np
import pytest

from oracle import river_oracle as O
from token_level_early_amd import configs, synth

pytestmark = pytest.mark.slow


def test_one_ulp_at_layer1_is_amplified_to_percent_level_logits():
    c = configs.model_cfg(configs.LLAMA_1B)
    L = c["L"]
    w = synth.to_numpy(synth.weights(c, seed=0, device="cpu"))
    mats = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")
    W = [{m: w["layers"][i][m].astype(np.float64) for m in mats} for i in range(L)]
    norms = [{"attn_norm": w["layers"][i]["attn_norm"], "mlp_norm": w["layers"][i]["mlp_norm"]}
             for i in range(L)]
    head = w["embed"].astype(np.float64)

    def run(tokens, perturb):
        K = np.zeros((L, c["Hkv"], len(tokens), c["D"]), np.float16)
        V = np.zeros_like(K)
        for pos, tok in enumerate(tokens):
            h = w["embed"][tok].copy()
            for l in range(L):
                h = O.block_decode(c, W[l], norms[l], h, pos, K[l], V[l])
                if l == 0 and pos == len(tokens) - 1 and perturb is not None:
                    h = h.copy()
                    h[perturb] = np.nextafter(h[perturb], np.float16(np.inf))
        x = O.rmsnorm(h, w["final_norm"], c["eps"]).astype(np.float64)
        return x @ head.T

    toks = synth.prompt(c, 1, 4, seed=0).numpy()[0]
    base = run(toks, None)
    pert = run(toks, np.array([5, 700]))  # two of 2048 elements
    rel = np.max(np.abs(base - pert)) / np.sqrt(np.mean(base * base))
    assert rel > 3e-3, rel  # the floor is a sizeable fraction of the 1e-2 per-block bound
