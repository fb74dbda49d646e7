"""The C-ABI library loads, exports every symbol include/river.h declares, and rejects bad
arguments before touching the GPU (host-only calls; no GPU needed)."""

import ctypes
import os
import re

import pytest

from token_level_early_amd import configs, river

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "river.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(river_\w+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol():
    lib = river.load()
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.parametrize("name", ["tiny", "llama3.2-1b-shape", "llama3.1-8b-shape"])
def test_kv_layout_is_one_backbone_sized_cache(name):
    c = configs.model_cfg(configs.ALL[name])
    Tmax = 1000
    d = river.kv_layout(river.make_config(c, Tmax))
    assert list(d.dims) == [c["L"], 2, 1, c["Hkv"], Tmax, c["D"]]
    assert d.strides[5] == 1 and d.strides[4] == c["D"] and d.strides[0] == 2 * c["Hkv"] * Tmax * c["D"]
    # exactly one KV set of the backbone's size: L * 2 * B * Hkv * Tmax * D fp16
    assert d.total_bytes == c["L"] * 2 * c["Hkv"] * Tmax * c["D"] * 2


def test_long_context_adds_no_second_kv_set():
    """The caller's cache is the only KV storage: raising max_seq from 1000 to 65600 positions
    (the 64K-prompt workload) grows the library's scratch only by the RoPE table (cos, sin per
    position and frequency, fp32), never by anything proportional to L * positions."""
    c = configs.model_cfg(configs.LLAMA_8B)
    t1, t2 = 1000, 65600
    _, s1 = river.workspace_bytes(river.make_config(c, t1, 512))
    _, s2 = river.workspace_bytes(river.make_config(c, t2, 512))
    rope = (t2 - t1) * (c["D"] // 2) * 8
    kv_growth = c["L"] * 2 * c["Hkv"] * (t2 - t1) * c["D"] * 2
    assert s2 - s1 <= rope + 4096, (s1, s2, rope)
    assert s2 - s1 <= kv_growth / 256  # the RoPE table: 512 B per position against 128 KiB of KV
    k1 = river.kv_layout(river.make_config(c, t1, 512)).total_bytes
    k2 = river.kv_layout(river.make_config(c, t2, 512)).total_bytes
    assert k2 - k1 == kv_growth


def test_river_buffer_covers_int4_copy():
    c = configs.model_cfg(configs.LLAMA_8B)
    rb, sb = river.workspace_bytes(river.make_config(c, 2400, 2048))
    P_l = 218_103_808
    assert c["L"] * (P_l // 2 + 2 * P_l // c["group"]) <= rb <= 1.01 * c["L"] * (P_l // 2 + 2 * P_l // c["group"])
    assert sb > 0


@pytest.mark.parametrize("field,value,msg", [
    ("n_kv_heads", 3, "multiple of n_kv_heads"),
    ("head_dim", 96, "head_dim"),
    ("group", 48, "group"),
    ("max_prefill", 5000, "max_prefill"),
    ("entry_layer", 0, "entry_layer"),
    ("entry_layer", 33, "entry_layer"),
    ("d_model", 4100, "d_model"),
    ("max_batch", 17, "max_batch"),
    ("max_batch", 0, "max_batch"),
    ("rms_eps", 0.0, "rms_eps"),
    ("zero_point", 2, "zero_point"),
])
def test_bad_config_rejected(field, value, msg):
    c = configs.model_cfg(configs.LLAMA_8B)
    cfg = river.make_config(c, 2400, 2048)
    setattr(cfg, field, value)
    with pytest.raises(river.RiverError) as e:
        river.kv_layout(cfg)
    assert e.value.code == river.RIVER_EINVAL and msg in str(e.value)


def test_init_rejects_null_arguments_before_any_device_work():
    lib = river.load()
    c = configs.model_cfg(configs.TINY)
    cfg = river.make_config(c, 128)
    ctx = ctypes.c_void_p()
    rc = lib.river_init(ctypes.byref(cfg), None, None, None, None, None, ctypes.byref(ctx))
    assert rc == river.RIVER_EINVAL and lib.river_last_error()
    w = river.Weights()
    rc = lib.river_init(ctypes.byref(cfg), ctypes.byref(w), ctypes.c_void_p(1), ctypes.c_void_p(1),
                        ctypes.c_void_p(1), None, ctypes.byref(ctx))
    assert rc == river.RIVER_EINVAL
    assert lib.river_destroy(None) == river.RIVER_OK
    assert lib.river_decode_path(None, None) == river.RIVER_EINVAL
    assert lib.river_decode_step(None, None, None, 0.5, None, None, None, None, None) == river.RIVER_EINVAL
    assert lib.river_prefill(None, None, 1, 0, 0.5, None, None, None, None, None) == river.RIVER_EINVAL


def test_kv_write_counting_only_in_the_debug_build():
    """river_kv_counting (host-only) reports 0 in the release library and 1 in the library built
    with RIVER_DEBUG_KV_COUNT; both export the same symbols."""
    flag = ctypes.c_int32(-1)
    assert river.load().river_kv_counting(ctypes.byref(flag)) == 0 and flag.value == 0
    dbg = river.load(river.LIB_KVCOUNT_PATH)
    flag = ctypes.c_int32(-1)
    assert dbg.river_kv_counting(ctypes.byref(flag)) == 0 and flag.value == 1
    for n in _declared():
        assert hasattr(dbg, n), n


def test_phase_trace_only_in_the_trace_build():
    """river_phase_trace (host-only copy) reports the timestamp array's shape in both libraries,
    refuses in the release one and copies in the one built with RIVER_PHASE_TRACE; both export
    the same symbols."""
    dims = (ctypes.c_int32 * 4)()
    assert river.load().river_phase_trace(None, 0, dims) == river.RIVER_EINVAL
    shape = tuple(dims)
    assert shape[2] == 10 and shape[3] >= 256 and shape[0] >= 8
    dbg = river.load(river.LIB_PHASETRACE_PATH)
    dims2 = (ctypes.c_int32 * 4)()
    assert dbg.river_phase_trace(None, 0, dims2) == 0 and tuple(dims2) == shape
    for n in _declared():
        assert hasattr(dbg, n), n


def test_prefill_scratch_is_bounded_by_the_chunk():
    """Prefill keeps the residual stream of every prompt row (2 x B*P*d fp16 plus one fp64
    similarity per row: the sequence-level exit needs all tokens of a layer before the next) and
    every other activation only for one chunk of positions: at the 64K-prompt workload the
    scratch is about 1.6 GB (1.07 GB of it the residual stream) instead of the 8.6 GB a
    whole-prompt layout needs, and beyond the residual stream it grows with the chunk, not with
    the prompt."""
    c = configs.model_cfg(configs.LLAMA_8B)
    d, hd, F, nqkv = c["d"], c["H"] * c["D"], c["F"], (c["H"] + 2 * c["Hkv"]) * c["D"]
    P = 65536
    per_row = 2 * (d + max(d, hd) + hd + nqkv + 2 * F + F)  # chunk activations, bytes per row
    sizes = {}
    for chunk in (1024, 4096):
        cfg = river.make_config(dict(c, prefill_chunk=chunk), P + 64, P)
        sizes[chunk] = river.workspace_bytes(cfg)[1]
    resid = 2 * P * d * 2 + P * 8
    assert abs((sizes[4096] - sizes[1024]) - 3072 * per_row) < 64 * 1024
    assert resid < sizes[4096] < resid + 4096 * per_row + (64 << 20)
    assert sizes[4096] < 1.7e9
    # the default chunk is 4096 positions of one row (4096 / max_batch per row)
    dflt = river.workspace_bytes(river.make_config(c, P + 64, P))[1]
    assert dflt == sizes[4096]
