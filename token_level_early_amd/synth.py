"""Seeded synthetic inputs: weights, prompts and exit schedules.

This module only draws random numbers; it holds none of the method's arithmetic.
Both the HIP path and the CPU oracle consume what it returns (the oracle receives
numpy copies), so neither side generates inputs for the other.

Streams: 0 = weights, 1 = prompt tokens, 2 = exit schedule. Each tensor gets its
own generator seeded from (cfg_id, stream, layer, tensor index, user seed).
"""

from __future__ import annotations

import numpy as np
import torch

_MATS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def _seed(*parts):
    h = 0x9E3779B97F4A7C15
    for p in parts:
        h = (h * 0x100000001B3 + (int(p) & 0xFFFFFFFFFFFF) + 0x632BE59BD9B4E019) % (1 << 63)
    return h


def _gen(device, *parts):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def _normal16(shape, std, device, *parts):
    g = _gen(device, *parts)
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(0.0, std, generator=g)
    return t.to(torch.float16)


def weight_shapes(c):
    d, H, Hkv, D, F = c["d"], c["H"], c["Hkv"], c["D"], c["F"]
    return {"wq": (H * D, d), "wk": (Hkv * D, d), "wv": (Hkv * D, d), "wo": (d, H * D),
            "w_gate": (F, d), "w_up": (F, d), "w_down": (d, F)}


def weights(c, seed=0, device="cpu", std=0.02, layers=None):
    """fp16 weights ~ N(0, std) (linear maps and embedding), RMSNorm gains = 1.

    Returns dict(embed, lm_head (None when tied), final_norm, layers=[dict ...]).
    ``layers`` limits which layer indices are generated (others are None).
    """
    cid = c.get("cfg_id", 0)
    shapes = weight_shapes(c)
    out = {"embed": _normal16((c["V"], c["d"]), std, device, cid, 0, 10000, 0, seed)}
    out["lm_head"] = None if c["tied"] else _normal16((c["V"], c["d"]), std, device,
                                                      cid, 0, 10001, 0, seed)
    out["final_norm"] = torch.ones(c["d"], dtype=torch.float16, device=device)
    lay = []
    for l in range(c["L"]):
        if layers is not None and l not in layers:
            lay.append(None)
            continue
        lw = {"attn_norm": torch.ones(c["d"], dtype=torch.float16, device=device),
              "mlp_norm": torch.ones(c["d"], dtype=torch.float16, device=device)}
        for ti, m in enumerate(_MATS):
            lw[m] = _normal16(shapes[m], std, device, cid, 0, l, ti + 1, seed)
        lay.append(lw)
    out["layers"] = lay
    return out


def representable_weights(c, seed=0, device="cpu", exp=-8):
    """Weights that int4 group quantisation reproduces exactly: every linear-map entry is
    q * 2^exp with integer q in [-7, 7] and at least one |q| = 7 in every group, so the
    group scale is exactly 2^exp. Embedding/LM head/norms as in ``weights``."""
    out = weights(c, seed=seed, device=device)
    g = c["group"]
    shapes = weight_shapes(c)
    for l, lw in enumerate(out["layers"]):
        for ti, m in enumerate(_MATS):
            N, K = shapes[m]
            gen = _gen(device, c.get("cfg_id", 0), 3, l, ti + 1, seed)
            q = torch.randint(-7, 8, (N, K), generator=gen, device=device, dtype=torch.int32)
            ng = (K + g - 1) // g
            for j in range(ng):
                col = j * g + torch.randint(0, min(g, K - j * g), (N,), generator=gen,
                                            device=device)
                sign = torch.where(torch.rand((N,), generator=gen, device=device) < 0.5, -7, 7)
                q[torch.arange(N, device=device), col] = sign.to(torch.int32)
            lw[m] = (q.to(torch.float32) * (2.0 ** exp)).to(torch.float16)
    return out


def prompt(c, B, P, seed=0, device="cpu"):
    """Prompt token ids ~ U[0, V), int32 [B][P]."""
    g = _gen(device, c.get("cfg_id", 0), 1, 0, 0, seed)
    return torch.randint(0, c["V"], (B, P), generator=g, device=device, dtype=torch.int32)


def schedule(c, S, B, seed=0, kind=None):
    """Forced exit layers int32 [S][B] (numpy), e = number of backbone layers.

    kind = ("uniform", lo, hi): e ~ U{lo..hi}; ("half", lo, hi): with probability 1/2
    e ~ U{lo..hi}, else e = L; ("const", e).
    """
    kind = kind or c.get("sched")
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [c.get("cfg_id", 0), 2, 0, 0, seed])))
    if kind[0] == "uniform":
        return rng.integers(kind[1], kind[2] + 1, size=(S, B)).astype(np.int32)
    if kind[0] == "half":
        e = rng.integers(kind[1], kind[2] + 1, size=(S, B))
        full = rng.random((S, B)) >= 0.5
        e[full] = c["L"]
        return e.astype(np.int32)
    if kind[0] == "const":
        return np.full((S, B), kind[1], dtype=np.int32)
    raise ValueError(kind)


def to_numpy(w):
    """Host numpy copies (fp16) of a weights dict, for the oracle."""
    def cv(t):
        return None if t is None else t.detach().cpu().numpy()
    out = {k: cv(w[k]) for k in ("embed", "lm_head", "final_norm")}
    out["layers"] = [None if lw is None else {k: cv(v) for k, v in lw.items()}
                     for lw in w["layers"]]
    return out


def representable_weights_zp(c, seed=0, device="cpu", exp=-8):
    """Weights that zero-point int4 group quantisation reproduces exactly: in every group the
    entries are (q - z0) * 2^exp with integer codes q in [0, 15], both q = 0 and q = 15 present,
    and one zero point z0 in [0, 15] per group, so the widened range is 15 * 2^exp and the
    group's scale is exactly 2^exp. Embedding/LM head/norms as in ``weights``."""
    out = weights(c, seed=seed, device=device)
    g = c["group"]
    shapes = weight_shapes(c)
    for l, lw in enumerate(out["layers"]):
        for ti, m in enumerate(_MATS):
            N, K = shapes[m]
            gen = _gen(device, c.get("cfg_id", 0), 4, l, ti + 1, seed)
            q = torch.randint(0, 16, (N, K), generator=gen, device=device, dtype=torch.int32)
            ng = (K + g - 1) // g
            z0 = torch.randint(0, 16, (N, ng), generator=gen, device=device, dtype=torch.int32)
            rows = torch.arange(N, device=device)
            for j in range(ng):
                w = min(g, K - j * g)
                c0 = j * g + torch.randint(0, w, (N,), generator=gen, device=device)
                c1 = j * g + (c0 - j * g + 1 + torch.randint(0, w - 1, (N,), generator=gen, device=device)) % w
                q[rows, c0] = 0
                q[rows, c1] = 15
            z = torch.repeat_interleave(z0, g, dim=1)[:, :K]
            lw[m] = ((q - z).to(torch.float32) * (2.0 ** exp)).to(torch.float16)
    return out
