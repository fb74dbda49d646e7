"""ctypes binding of libriver.so (include/river.h). Argument marshalling only: every step of
prefill and decode runs in the library's HIP kernels; torch provides device memory and the
stream. Fails loudly if the library is not built."""

from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libriver.so")
# the same library built with per-element KV write counters (RIVER_DEBUG_KV_COUNT; tests only)
LIB_KVCOUNT_PATH = os.path.join(_HERE, "libriver_kvcount.so")
# the same library with the persistent kernel recording phase timestamps (profiling only)
LIB_PHASETRACE_PATH = os.path.join(_HERE, "libriver_phasetrace.so")

RIVER_OK, RIVER_EINVAL, RIVER_ENOMEM, RIVER_ERANGE, RIVER_EHIP, RIVER_EDEVICE = 0, -1, -2, -3, -4, -5

MATS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


class RiverError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"river error {code}: {msg}")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("d_ffn", ctypes.c_int32),
        ("vocab", ctypes.c_int32), ("tied_embeddings", ctypes.c_int32), ("rms_eps", ctypes.c_float),
        ("rope_theta", ctypes.c_float), ("group", ctypes.c_int32), ("max_batch", ctypes.c_int32),
        ("max_seq", ctypes.c_int32), ("max_prefill", ctypes.c_int32), ("entry_layer", ctypes.c_int32),
        ("prefill_chunk", ctypes.c_int32), ("zero_point", ctypes.c_int32),
    ]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")]


class Weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("final_norm", ctypes.c_void_p), ("layers", ctypes.POINTER(LayerWeights))]


class KVDesc(ctypes.Structure):
    _fields_ = [("dims", ctypes.c_int64 * 6), ("strides", ctypes.c_int64 * 6),
                ("elem_bytes", ctypes.c_int32), ("total_bytes", ctypes.c_uint64)]


_libs = {}


def load(path=LIB_PATH):
    """Open libriver.so, or another build of it (raises if it is missing: there is no
    fallback path)."""
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    P, I32, F32, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
    sig = {
        "river_kv_layout": [P(Config), P(KVDesc)],
        "river_workspace_bytes": [P(Config), P(ctypes.c_uint64), P(ctypes.c_uint64)],
        "river_init": [P(Config), P(Weights), VP, VP, VP, VP, P(VP)],
        "river_destroy": [VP],
        "river_prefill": [VP, VP, I32, I32, F32, VP, VP, VP, VP, VP],
        "river_decode_step": [VP, VP, VP, F32, VP, VP, VP, VP, VP],
        "river_decode_steps": [VP, VP, VP, I32, F32, VP, VP, VP, VP],
        "river_decode_steps_static": [VP, VP, VP, I32, F32, VP, VP, VP, VP],
        "river_positions": [VP, P(I32)],
        "river_decode_path": [VP, P(I32)],
        "river_device_status": [VP, VP],
        "river_export_river": [VP, I32, I32, VP, VP, VP, VP],
        "river_debug_hidden": [VP, VP, VP],
        "river_decode_backbone_steps": [VP, VP, I32, VP, VP],
        "river_timer_arm": [VP, I32, I32],
        "river_timer_read": [VP, P(F32), P(I32)],
        "river_kv_write_counts": [VP, VP, VP],
        "river_weight_residency": [VP, P(ctypes.c_uint64), P(ctypes.c_uint64), P(ctypes.c_uint64)],
        "river_weight_placement": [VP, P(I32)],
        "river_kv_counting": [P(I32)],
        "river_phase_trace": [VP, ctypes.c_uint64, P(I32)],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.river_last_error.argtypes = []
    lib.river_last_error.restype = ctypes.c_char_p
    _libs[path] = lib
    return lib


def _check(rc, lib=None):
    if rc != RIVER_OK:
        raise RiverError(rc, (lib or load()).river_last_error().decode())


def make_config(c, max_seq, max_prefill=None, batch=1):
    """river_config from a model dict (see configs.model_cfg)."""
    return Config(n_layers=c["L"], d_model=c["d"], n_heads=c["H"], n_kv_heads=c["Hkv"],
                  head_dim=c["D"], d_ffn=c["F"], vocab=c["V"], tied_embeddings=int(c["tied"]),
                  rms_eps=c["eps"], rope_theta=c["theta"], group=c["group"], max_batch=batch,
                  max_seq=max_seq, max_prefill=max_prefill or max_seq,
                  entry_layer=c.get("entry", 1), prefill_chunk=int(c.get("prefill_chunk", 0)),
                  zero_point=int(bool(c.get("zero_point", False))))


def kv_layout(cfg: Config) -> KVDesc:
    d = KVDesc()
    _check(load().river_kv_layout(ctypes.byref(cfg), ctypes.byref(d)))
    return d


def workspace_bytes(cfg: Config):
    r, s = ctypes.c_uint64(), ctypes.c_uint64()
    _check(load().river_workspace_bytes(ctypes.byref(cfg), ctypes.byref(r), ctypes.byref(s)))
    return r.value, s.value


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class River:
    """One context: the borrowed fp16 backbone (torch tensors on the GPU), and torch-owned
    KV cache, river and scratch buffers sized by the library."""

    def __init__(self, c, weights, max_seq, max_prefill=None, batch=1, device="cuda",
                 lib_path=LIB_PATH, offload_from=None):
        """offload_from: backbone blocks with 0-based index >= offload_from are copied to
        page-locked host memory and handed to the library there (backbone offloading); the
        caller's device copies are not touched."""
        self.lib = load(lib_path)
        self.c = dict(c)
        self.cfg = make_config(c, max_seq, max_prefill, batch)
        self.B = batch
        self.w = weights
        self.kvdesc = kv_layout(self.cfg)
        r_, s_ = ctypes.c_uint64(), ctypes.c_uint64()
        self._chk(self.lib.river_workspace_bytes(ctypes.byref(self.cfg), ctypes.byref(r_),
                                                 ctypes.byref(s_)))
        rb, sb = r_.value, s_.value
        dev = torch.device(device)
        self.kv = torch.zeros(self.kvdesc.total_bytes // 2, dtype=torch.float16, device=dev)
        self.river_buf = torch.empty(rb, dtype=torch.uint8, device=dev)
        self.scratch = torch.empty(sb, dtype=torch.uint8, device=dev)
        L = c["L"]
        self._lw = (LayerWeights * L)()
        self._host = []  # page-locked copies of offloaded backbone blocks (kept alive here)
        for i, lw in enumerate(weights["layers"]):
            for n in ("attn_norm", "mlp_norm") + MATS:
                t = lw[n]
                assert t.is_cuda and t.dtype == torch.float16 and t.is_contiguous(), n
                if offload_from is not None and i >= offload_from and n in MATS:
                    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
                    h.copy_(t)
                    self._host.append(h)
                    t = h
                setattr(self._lw[i], n, t.data_ptr())
        self._w = Weights(embed=weights["embed"].data_ptr(),
                          lm_head=None if weights["lm_head"] is None else weights["lm_head"].data_ptr(),
                          final_norm=weights["final_norm"].data_ptr(),
                          layers=ctypes.cast(self._lw, ctypes.POINTER(LayerWeights)))
        ctx = ctypes.c_void_p()
        self._chk(self.lib.river_init(ctypes.byref(self.cfg), ctypes.byref(self._w), _ptr(self.kv),
                                   _ptr(self.river_buf), _ptr(self.scratch), _stream(),
                                   ctypes.byref(ctx)))
        self.ctx = ctx

    def _chk(self, rc):
        _check(rc, self.lib)

    def close(self):
        if self.ctx:
            self._chk(self.lib.river_destroy(self.ctx))
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- views
    def kv_view(self):
        """The shared cache as [L][2][B][Hkv][Tmax][D] fp16."""
        return self.kv.view(*[int(x) for x in self.kvdesc.dims])

    def positions(self):
        arr = (ctypes.c_int32 * self.B)()
        self._chk(self.lib.river_positions(self.ctx, arr))
        return list(arr)

    def residency(self):
        """Bytes of the borrowed weights in device and in host memory, and of the river."""
        d, h, r = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
        self._chk(self.lib.river_weight_residency(self.ctx, ctypes.byref(d), ctypes.byref(h), ctypes.byref(r)))
        return {"device_bytes": d.value, "host_bytes": h.value, "river_bytes": r.value}

    def decode_path(self):
        """"persistent" or "per_op": the kernels that serve this context's decode calls."""
        v = ctypes.c_int32()
        self._chk(self.lib.river_decode_path(self.ctx, ctypes.byref(v)))
        return "persistent" if v.value else "per_op"

    def device_status(self):
        return self.lib.river_device_status(self.ctx, _stream())

    # ---- calls
    def prefill(self, tokens, prefill_exit=0, tau=float("nan"), logits=False, min_sim=False):
        dev = tokens.device
        tokens = tokens.to(torch.int32).contiguous()
        B, P = tokens.shape
        nt = torch.empty(B, dtype=torch.int32, device=dev)
        lg = torch.empty(B, self.c["V"], dtype=torch.float32, device=dev) if logits else None
        se = torch.empty(B, dtype=torch.int32, device=dev)
        ms = torch.empty(B, self.c["L"], dtype=torch.float32, device=dev) if min_sim else None
        self._chk(self.lib.river_prefill(self.ctx, _ptr(tokens), P, int(prefill_exit), float(tau),
                                      _ptr(nt), _ptr(lg), _ptr(se), _ptr(ms), _stream()))
        return {"tokens": nt, "logits": lg, "seq_exit": se, "min_sim": ms}

    def decode_step(self, tok_in, forced_exit=None, tau=float("nan"), logits=False, sim=True):
        dev = tok_in.device
        tok_in = tok_in.to(torch.int32).contiguous()
        fe = None if forced_exit is None else forced_exit.to(torch.int32).contiguous()
        out = torch.empty(self.B, dtype=torch.int32, device=dev)
        ex = torch.empty(self.B, dtype=torch.int32, device=dev)
        lg = torch.empty(self.B, self.c["V"], dtype=torch.float32, device=dev) if logits else None
        sm = torch.empty(self.B, self.c["L"], dtype=torch.float32, device=dev) if sim else None
        self._chk(self.lib.river_decode_step(self.ctx, _ptr(tok_in), _ptr(fe), float(tau), _ptr(out),
                                          _ptr(lg), _ptr(ex), _ptr(sm), _stream()))
        return {"tokens": out, "logits": lg, "exit_layer": ex, "sim": sm}

    def decode_steps(self, tok_in, sched=None, S=None, tau=float("nan"), tok_out=None,
                     exit_layer=None, sim=None):
        """S steps on the device. sched [S][B] int32 (forced) or None (tau mode)."""
        dev = tok_in.device
        if sched is not None:
            S = sched.shape[0]
        if tok_out is None:
            tok_out = torch.empty(S, self.B, dtype=torch.int32, device=dev)
        self._chk(self.lib.river_decode_steps(self.ctx, _ptr(tok_in), _ptr(sched), int(S), float(tau),
                                           _ptr(tok_out), _ptr(exit_layer), _ptr(sim), _stream()))
        return tok_out

    def decode_steps_static(self, tok_in, sched=None, S=None, tau=float("nan"), tok_out=None,
                            exit_layer=None, sim=None):
        """decode_steps with the exchange buffers in the library's fixed device array
        (river_decode_steps_static: no allocation inside the call)."""
        dev = tok_in.device
        if sched is not None:
            S = sched.shape[0]
        if tok_out is None:
            tok_out = torch.empty(S, self.B, dtype=torch.int32, device=dev)
        self._chk(self.lib.river_decode_steps_static(self.ctx, _ptr(tok_in), _ptr(sched), int(S), float(tau),
                                                     _ptr(tok_out), _ptr(exit_layer), _ptr(sim), _stream()))
        return tok_out

    def decode_backbone_steps(self, tok_in, S, tok_out=None):
        """S full-depth fp16 steps (backbone only, no exit test)."""
        if tok_out is None:
            tok_out = torch.empty(S, self.B, dtype=torch.int32, device=tok_in.device)
        self._chk(self.lib.river_decode_backbone_steps(self.ctx, _ptr(tok_in), int(S), _ptr(tok_out),
                                                    _stream()))
        return tok_out

    TIMER_OPS = {"qkv": 0, "attn": 1, "o": 2, "gu": 3, "down": 4, "lm": 5, "persist": 6}

    def timer_arm(self, op, max_launches):
        self._chk(self.lib.river_timer_arm(self.ctx, self.TIMER_OPS[op], int(max_launches)))

    def timer_read(self, max_launches):
        """Per-launch durations (ms) of the armed op, in launch order."""
        buf = (ctypes.c_float * max_launches)()
        n = ctypes.c_int32(max_launches)
        self._chk(self.lib.river_timer_read(self.ctx, buf, ctypes.byref(n)))
        return list(buf[: n.value])

    def export_river(self, layer, which):
        """Canonical packed nibbles [N][ceil(K/2)] uint8 and scales [N][ceil(K/g)] fp16, plus the
        zero points [N][ceil(K/g)] uint8 for the zero-point format (a third return value)."""
        c = self.c
        shapes = {"wq": (c["H"] * c["D"], c["d"]), "wk": (c["Hkv"] * c["D"], c["d"]),
                  "wv": (c["Hkv"] * c["D"], c["d"]), "wo": (c["d"], c["H"] * c["D"]),
                  "w_gate": (c["F"], c["d"]), "w_up": (c["F"], c["d"]), "w_down": (c["d"], c["F"])}
        N, K = shapes[MATS[which]]
        packed = torch.empty(N, (K + 1) // 2, dtype=torch.uint8, device=self.kv.device)
        scales = torch.empty(N, math.ceil(K / c["group"]), dtype=torch.int16, device=self.kv.device)
        zp = bool(c.get("zero_point", False))
        zeros = torch.empty(N, math.ceil(K / c["group"]), dtype=torch.uint8, device=self.kv.device) if zp else None
        self._chk(self.lib.river_export_river(self.ctx, int(layer), int(which), _ptr(packed),
                                              _ptr(scales), _ptr(zeros), _stream()))
        if zp:
            return packed, scales.view(torch.float16), zeros
        return packed, scales.view(torch.float16)

    def kv_write_counts(self):
        """Writes per shared-cache slot, uint8 [L][B][max_seq] (255: the slot's elements were
        written unequal numbers of times). Needs the library built with RIVER_DEBUG_KV_COUNT."""
        c = self.c
        out = torch.empty(c["L"], self.B, int(self.kvdesc.dims[4]), dtype=torch.uint8,
                          device=self.kv.device)
        self._chk(self.lib.river_kv_write_counts(self.ctx, _ptr(out), _stream()))
        return out

    def phase_trace(self):
        """Phase timestamps of the last persistent launch, uint64 [steps][slots][events][workgroups]
        (100 MHz ticks). Needs the library built with RIVER_PHASE_TRACE."""
        import numpy as np
        dims = (ctypes.c_int32 * 4)()
        self._chk(self.lib.river_phase_trace(None, 0, dims))
        shape = tuple(int(x) for x in dims)
        out = np.zeros(shape, dtype=np.uint64)
        self._chk(self.lib.river_phase_trace(out.ctypes.data_as(ctypes.c_void_p), out.size, dims))
        return out

    def hidden(self):
        """Residual stream of the last decode step: [L+1][B][d] fp16."""
        c = self.c
        out = torch.empty(c["L"] + 1, self.B, c["d"], dtype=torch.float16, device=self.kv.device)
        self._chk(self.lib.river_debug_hidden(self.ctx, _ptr(out), _stream()))
        return out
