"""Backbone offloading (paperlayer.ai summary of arXiv 2604.18396v3, section 4 "Deployment
Efficiency" and appendix A.3; aitrends.kr offloading paragraph): backbone blocks past a depth
live in page-locked host memory and are read over the host link only by tokens that still run
them. The library reports where the parameters are, and an offloaded context decodes exactly
like a resident one -- same kernels, same bits -- for schedules that cross the offload depth,
on the persistent, per-op and batched paths."""

import ctypes
import os

import numpy as np
import pytest
import torch

from token_level_early_amd import configs, river, synth
from tests._util import f32

pytestmark = pytest.mark.gpu

TINY = configs.model_cfg(configs.TINY)


def _ctx(c, w, path, batch, offload_from, **kw):
    old = os.environ.get("RIVER_PERSIST")
    os.environ["RIVER_PERSIST"] = "1" if path == "persistent" else "0"
    try:
        return river.River(c, w, batch=batch, offload_from=offload_from, **kw)
    finally:
        if old is None:
            del os.environ["RIVER_PERSIST"]
        else:
            os.environ["RIVER_PERSIST"] = old


def _layer_bytes(c):
    d, hd, kvd, F = c["d"], c["H"] * c["D"], c["Hkv"] * c["D"], c["F"]
    return 2 * (hd * d + 2 * kvd * d + d * hd + 3 * F * d)


@pytest.mark.parametrize("path,batch", [("persistent", 1), ("per_op", 1), ("batched", 3)])
def test_offloaded_backbone_decodes_like_resident(path, batch):
    c = TINY
    L, P, S, R = c["L"], 12, 10, 2  # blocks 3 and 4 (0-based 2, 3) offloaded
    w = synth.weights(c, seed=0, device="cuda")
    rng = np.random.default_rng(5)
    sched = torch.from_numpy(rng.integers(0, L + 1, size=(S, batch)).astype(np.int32)).cuda()
    sched[0, 0], sched[1, 0] = L, 3  # tokens that run offloaded blocks
    toks = synth.prompt(c, batch, P, seed=9, device="cuda")
    out = []
    for off in (None, R):
        rv = _ctx(c, w, "persistent" if path == "persistent" else "per_op", batch, off,
                  max_seq=P + S + 4, max_prefill=P)
        res = rv.residency()
        if off is None:
            assert res["host_bytes"] == 0
        else:
            assert res["host_bytes"] == (L - R) * _layer_bytes(c)
        pre = rv.prefill(toks, prefill_exit=L)
        ex = torch.empty(S, batch, dtype=torch.int32, device="cuda")
        t = rv.decode_steps(pre["tokens"], sched=sched, exit_layer=ex)
        t2 = rv.decode_steps(t[-1].clone(), S=3, tau=f32(0.5))
        torch.cuda.synchronize()
        assert rv.device_status() == river.RIVER_OK
        out.append((pre["tokens"].cpu(), t.cpu(), ex.cpu(), t2.cpu(), rv.kv_view().cpu(), rv.hidden().cpu(),
                    res))
        rv.close()
    a, b = out
    assert b[6]["device_bytes"] + b[6]["host_bytes"] == a[6]["device_bytes"]
    assert b[6]["river_bytes"] == a[6]["river_bytes"]
    for x, y in zip(a[:6], b[:6]):
        assert torch.equal(x, y)


def test_pageable_host_weights_are_rejected():
    c = TINY
    w = synth.weights(c, seed=0, device="cuda")
    lib = river.load()
    cfg = river.make_config(c, 16)
    lw = (river.LayerWeights * c["L"])()
    pageable = np.zeros(c["F"] * c["d"], np.float16)  # ordinary host memory
    for i, l in enumerate(w["layers"]):
        for n in ("attn_norm", "mlp_norm") + river.MATS:
            setattr(lw[i], n, l[n].data_ptr())
    lw[1].w_up = pageable.ctypes.data
    kind = ctypes.c_int32(-1)
    # the library's own classification (no device work): pinned host accepted, pageable refused
    pin = torch.empty(16, dtype=torch.float16, pin_memory=True)
    assert lib.river_weight_placement(ctypes.c_void_p(pin.data_ptr()), ctypes.byref(kind)) == 0 and kind.value == 1
    assert lib.river_weight_placement(ctypes.c_void_p(w["embed"].data_ptr()), ctypes.byref(kind)) == 0 and kind.value == 0
    assert lib.river_weight_placement(ctypes.c_void_p(pageable.ctypes.data), ctypes.byref(kind)) == river.RIVER_EINVAL
    ws = river.Weights(embed=w["embed"].data_ptr(), lm_head=w["lm_head"].data_ptr(),
                       final_norm=w["final_norm"].data_ptr(),
                       layers=ctypes.cast(lw, ctypes.POINTER(river.LayerWeights)))
    kvb = river.kv_layout(cfg).total_bytes
    rb, sb = river.workspace_bytes(cfg)
    kv = torch.zeros(kvb // 2, dtype=torch.float16, device="cuda")
    rbuf = torch.empty(rb, dtype=torch.uint8, device="cuda")
    sbuf = torch.empty(sb, dtype=torch.uint8, device="cuda")
    ctx = ctypes.c_void_p()
    rc = lib.river_init(ctypes.byref(cfg), ctypes.byref(ws), ctypes.c_void_p(kv.data_ptr()),
                        ctypes.c_void_p(rbuf.data_ptr()), ctypes.c_void_p(sbuf.data_ptr()),
                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), ctypes.byref(ctx))
    assert rc == river.RIVER_EINVAL
    assert b"layer 1 w_up" in lib.river_last_error()
    torch.cuda.synchronize()
