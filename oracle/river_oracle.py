"""Plain, slow CPU oracle of River-LLM token-level early-exit decode (NumPy, fp64).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.

Pages this follows (all about "River-LLM: Large Language Model Seamless Exit Based
on KV Share", Shen & Zou):
  [paperlayer]  paperlayer.ai summary of arXiv 2604.18396v3, sections §3 Motivation,
                §4 Seamless Exit: River-LLM, §5 Evaluation, A.3 Detailed Memory Usage.
  [aitrends]    aitrends.kr article "River-LLM: KV 공유 기반의 대형 언어 모델 심리스
                조기 종료 기법": the paragraphs on the exit-layer construction, the exit
                criterion, prefill vs generation, and the KV-share mechanism.
  [chatpaper]   chatpaper.ai abstract page (problem statement: KV Cache Absence).

What the method computes, per the pages:
  * Each backbone decoder block has a plug-in exit layer ("exit river" layer) that is a
    copy of that block's weights quantised to 4-bit weights with 16-bit activations
    (W4A16) [aitrends, construction paragraph; paperlayer §4 KV-Shared Exit Layer].
  * Exit layers use the backbone's KV addressing and an fp16 KV cache, so the KV a
    token produces on the river lands in the same slots the backbone would have
    filled; there is one KV set [paperlayer §4 KV-Shared Exit Layer, A.3;
    aitrends, KV-share paragraph].
  * The exit test is the cosine similarity between a block's input h(l-1) and its
    output h(l) (dot product, then normalised by the magnitudes); the token exits
    when it is larger than tau [aitrends, exit-criterion paragraph; paperlayer §4
    Error-Aware Exit Decisions].
  * After an exit the remaining layers run on the serial exit layers and the
    original LM head produces the logits [paperlayer §4 Inference with Seamless Exit].
  * Prefill uses one exit depth for the whole sequence; generation exits per token
    [paperlayer §4 Inference with Seamless Exit; aitrends, prefill paragraph;
    paperlayer §3 Sequence-level Exit: the latest-exiting token sets the depth].

Readings taken where the pages are silent:
  R1  h(l-1), h(l) are the residual-stream vectors entering/leaving block l, as
      stored (fp16), not normalised.
  R2  strict comparison s > tau.
  R3  the test runs after backbone layers l in [E_min, L-1]; nothing is tested after
      a river layer or after layer L. Default E_min = 1.
  R4  exits are monotone: once a token leaves the backbone at layer e, layers
      e+1..L all run on the river (none are skipped).
  R5  quantiser (the pages name HQQ/AWQ but give no formula): symmetric round-to-
      nearest int4 per group of ``group`` consecutive input columns; scale
      s = fp16(fp32(amax/7)); q = clamp(rint(fp32(w/s)), -8, 7) (round half to
      even); s == 0 gives q = 0; dequantised weight q*s is exact.  Stored nibble
      u = q + 8, element 2i in the low nibble of byte i.
  R5z the zero-point river format (the pages' alternative backends, HQQ and AWQ, store a
      scale and a zero point per group; their calibration is not reproduced): asymmetric
      round-to-nearest int4 per group with the range widened to hold 0:
      lo = min(min w, 0), hi = max(max w, 0) (fp16 values, so hi - lo is exact in fp64),
      s = fp16(fp32((hi - lo) / 15)); s == 0 gives q = 0 and z = 0; else
      z = clamp(rint(fp32(-lo / s)), 0, 15) and q = clamp(rint(fp32(w / s)) + z, 0, 15)
      (round half to even); dequantised weight (q - z)*s is exact.  Stored nibble u = q,
      element 2i in the low nibble of byte i; zero points one byte per group.
  R6  the seven linear maps of a block are quantised; RMSNorm gains, embedding and
      LM head stay fp16.
  R7  river layer l reads and writes the same KV[l] as backbone layer l.
  R8  prefill (tau mode): the sequence exits after backbone layer l iff
      min over prompt tokens of s_t(l) > tau; forced mode exits at the given layer.
  R9  Llama-style block: RMSNorm (eps) -> QKV -> rotate-half RoPE -> GQA attention
      (kv head = q head // (H/Hkv)) -> O + residual -> RMSNorm -> SwiGLU -> down +
      residual.
  R10 zero-norm cosine is 0.
  R11 greedy argmax takes the lowest index on ties.

Precision: arithmetic in fp64; values are rounded to fp16 (round to nearest even)
where the pages fix fp16 storage (activations between ops, KV cache), see
``block_decode``.  The quantiser's divisions are the fp32 IEEE divisions of R5.

Parity notes: every function here is pinned by tests/test_oracle_*.py against
closed forms, invariants or brute force; the whole-decoder composition (logits) has
no printed example on the pages and is pinned only through those primitives and the
identities in tests/test_oracle_decode.py.
"""

from __future__ import annotations

import numpy as np

F16 = np.float16
F32 = np.float32
F64 = np.float64


def to_f16(x):
    """Round to IEEE binary16 with round-to-nearest-even (the fp16 storage points)."""
    return np.asarray(x).astype(F16)


def argmax_lowest(x):
    """Greedy token: index of the maximum, lowest index on ties (reading R11)."""
    x = np.asarray(x)
    return int(np.flatnonzero(x == x.max())[0])


# --------------------------------------------------------------------------------------
# W4A16 river construction (reading R5; [aitrends] construction paragraph,
# [paperlayer] §4 KV-Shared Exit Layer: 4-bit weight-only quantisation)
# --------------------------------------------------------------------------------------

def quantize_w4(W16, group):
    """Quantise an fp16 matrix W[N][K] to int4 codes q[N][K] and fp16 scales s[N][ceil(K/group)].

    Groups run along K (the input dimension); the last group of a row may be short.
    """
    W = np.asarray(W16, dtype=F16).astype(F32)
    N, K = W.shape
    ng = (K + group - 1) // group
    q = np.zeros((N, K), dtype=np.int8)
    scales = np.zeros((N, ng), dtype=F16)
    for j in range(ng):
        lo, hi = j * group, min((j + 1) * group, K)
        blk = W[:, lo:hi]
        amax = np.abs(blk).max(axis=1)                      # exact in fp32
        s16 = (amax / F32(7.0)).astype(F32).astype(F16)     # IEEE fp32 divide, then RNE to fp16
        s32 = s16.astype(F32)
        zero = s32 == 0
        denom = np.where(zero, F32(1.0), s32).astype(F32)
        r = np.rint(blk / denom[:, None]).astype(F32)       # IEEE fp32 divide, round half to even
        r[zero, :] = 0
        q[:, lo:hi] = np.clip(r, -8, 7).astype(np.int8)
        scales[:, j] = s16
    return q, scales


def quantize_w4_zp(W16, group):
    """Asymmetric int4 with an integer zero point per group (reading R5z): codes q[N][K] in
    [0, 15] (uint8), fp16 scales s[N][ceil(K/group)], zero points z[N][ceil(K/group)] (uint8)."""
    W = np.asarray(W16, dtype=F16).astype(F32)
    N, K = W.shape
    ng = (K + group - 1) // group
    q = np.zeros((N, K), dtype=np.uint8)
    scales = np.zeros((N, ng), dtype=F16)
    zeros = np.zeros((N, ng), dtype=np.uint8)
    for j in range(ng):
        c0, c1 = j * group, min((j + 1) * group, K)
        blk = W[:, c0:c1]
        lo = np.minimum(blk.min(axis=1), F32(0.0)).astype(F64)
        hi = np.maximum(blk.max(axis=1), F32(0.0)).astype(F64)
        s16 = ((hi - lo) / 15.0).astype(F32).astype(F16)   # exact range, fp32 then fp16 rounding
        s32 = s16.astype(F32)
        zero = s32 == 0
        denom = np.where(zero, F32(1.0), s32).astype(F32)
        z = np.clip(np.rint((-lo).astype(F32) / denom), 0, 15).astype(F32)   # fp32 divide, RNE
        r = np.rint(blk / denom[:, None]).astype(F32) + z[:, None]
        r[zero, :] = 0
        z[zero] = 0
        q[:, c0:c1] = np.clip(r, 0, 15).astype(np.uint8)
        scales[:, j] = s16
        zeros[:, j] = z.astype(np.uint8)
    return q, scales, zeros


def dequantize_w4_zp(q, scales, zeros, group):
    """Zero-point river weight W^[n][k] = (q[n][k] - z[n][k // group]) * s[n][k // group], exact
    in fp64."""
    q = np.asarray(q)
    N, K = q.shape
    s = np.repeat(np.asarray(scales).astype(F64), group, axis=1)[:, :K]
    z = np.repeat(np.asarray(zeros).astype(F64), group, axis=1)[:, :K]
    return (q.astype(F64) - z) * s


def pack_codes(u):
    """Unsigned 4-bit codes u[N][K] packed two per byte, element 2i in the low nibble of byte i
    (odd K pads a 0 nibble): the zero-point format's code layout."""
    u = np.asarray(u, dtype=np.uint8)
    N, K = u.shape
    if K % 2:
        u = np.concatenate([u, np.zeros((N, 1), np.uint8)], axis=1)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def pack_nibbles(q):
    """Offset-binary nibbles u = q + 8, element 2i in the low nibble of byte i (odd K pads u=8)."""
    q = np.asarray(q, dtype=np.int16)
    N, K = q.shape
    u = (q + 8).astype(np.uint8)
    if K % 2:
        u = np.concatenate([u, np.full((N, 1), 8, np.uint8)], axis=1)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed, K):
    """Inverse of pack_nibbles: int4 codes q[N][K]."""
    packed = np.asarray(packed, dtype=np.uint8)
    N, nb = packed.shape
    u = np.empty((N, 2 * nb), dtype=np.int16)
    u[:, 0::2] = packed & 0x0F
    u[:, 1::2] = packed >> 4
    return (u[:, :K] - 8).astype(np.int8)


def dequantize_w4(q, scales, group):
    """River weight W^[n][k] = q[n][k] * s[n][k // group], exact in fp64."""
    q = np.asarray(q)
    N, K = q.shape
    s = np.repeat(np.asarray(scales).astype(F64), group, axis=1)[:, :K]
    return q.astype(F64) * s


# --------------------------------------------------------------------------------------
# Block primitives (reading R9)
# --------------------------------------------------------------------------------------

def rmsnorm(h16, w16, eps):
    """fp16( h / sqrt(mean(h^2) + eps) * w ), computed in fp64 along the last axis."""
    h = np.asarray(h16).astype(F64)
    inv = 1.0 / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    return to_f16(h * inv * np.asarray(w16).astype(F64))


def rope_cos_sin(pos, D, theta):
    """cos/sin of pos * theta^(-2i/D), i < D/2, in fp64. pos may be a scalar or a vector."""
    i = np.arange(D // 2, dtype=F64)
    inv_freq = np.power(F64(theta), -2.0 * i / D)
    ang = np.multiply.outer(np.asarray(pos, dtype=F64), inv_freq)
    return np.cos(ang), np.sin(ang)


def apply_rope(x16, cos, sin):
    """Rotate-half RoPE: pairs (i, i + D/2) rotate by angle_i. x16 [..., D]; cos/sin broadcast
    against [..., D/2]. Result rounded to fp16."""
    x = np.asarray(x16).astype(F64)
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    return to_f16(np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1))


def cosine(a16, b16):
    """State-transition similarity s = <a,b> / (|a| |b|) in fp64 ([aitrends] exit-criterion
    paragraph: dot product, then normalisation by the magnitudes). Zero norm gives 0 (R10)."""
    a = np.asarray(a16).astype(F64).ravel()
    b = np.asarray(b16).astype(F64).ravel()
    na = np.sqrt(np.dot(a, a))
    nb = np.sqrt(np.dot(b, b))
    if na == 0.0 or nb == 0.0:
        return 0.0
    return float(np.dot(a, b) / (na * nb))


def silu(x):
    x = np.asarray(x, dtype=F64)
    return x / (1.0 + np.exp(-x))


def _softmax_rows(s):
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=-1, keepdims=True)


def decode_attention(q16, K16, V16):
    """One query position. q16 [H][D]; K16, V16 [Hkv][T][D] (the shared cache, positions
    0..T-1). Query head h reads KV head h // (H/Hkv). Returns o [H][D] fp16."""
    H, D = q16.shape
    Hkv = K16.shape[0]
    G = H // Hkv
    o = np.empty((H, D), dtype=F16)
    for h in range(H):
        kv = h // G
        k = np.asarray(K16[kv]).astype(F64)
        v = np.asarray(V16[kv]).astype(F64)
        s = (k @ q16[h].astype(F64)) / np.sqrt(F64(D))
        p = _softmax_rows(s[None, :])[0]
        o[h] = to_f16(p @ v)
    return o


def causal_attention(Q16, K16, V16):
    """Prompt attention. Q16 [P][H][D]; K16, V16 [Hkv][P][D]. Position t attends to 0..t.
    Returns O [P][H][D] fp16."""
    P, H, D = Q16.shape
    Hkv = K16.shape[0]
    G = H // Hkv
    O = np.empty((P, H, D), dtype=F16)
    mask = np.triu(np.ones((P, P), dtype=bool), k=1)
    for h in range(H):
        kv = h // G
        k = np.asarray(K16[kv]).astype(F64)
        v = np.asarray(V16[kv]).astype(F64)
        s = (Q16[:, h, :].astype(F64) @ k.T) / np.sqrt(F64(D))
        s[mask] = -np.inf
        O[:, h, :] = to_f16(_softmax_rows(s) @ v)
    return O


def _lin(W, x16):
    """x16 [..., K] (fp16) times W[N][K]^T in fp64 (not rounded)."""
    return np.asarray(x16).astype(F64) @ np.asarray(W).T


# --------------------------------------------------------------------------------------
# Shared KV cache (one set, backbone addressing: [paperlayer] §4, A.3; [aitrends] KV share)
# --------------------------------------------------------------------------------------

class OracleKV:
    """K and V caches [L][B][Hkv][Tmax][D] fp16 plus a write counter [L][B][Tmax].

    Both the backbone block and its river copy write layer l's slot at the token's
    position; the counter lets tests check that every (layer, position) slot is written
    exactly once whatever the exit schedule (the KV Cache Absence problem of
    [chatpaper] abstract / [paperlayer] §3 is then absent).
    """

    def __init__(self, L, B, Hkv, Tmax, D):
        self.K = np.zeros((L, B, Hkv, Tmax, D), dtype=F16)
        self.V = np.zeros((L, B, Hkv, Tmax, D), dtype=F16)
        self.count = np.zeros((L, B, Tmax), dtype=np.int32)
        self.pos = np.zeros(B, dtype=np.int64)

    def write(self, l, b, pos, k16, v16):
        self.K[l, b, :, pos, :] = k16
        self.V[l, b, :, pos, :] = v16
        self.count[l, b, pos] += 1


# --------------------------------------------------------------------------------------
# One decoder block (backbone or river: same code, different weight matrices)
# --------------------------------------------------------------------------------------

def block_decode(cfg, W, norms, h_in16, pos, K_l, V_l, trace=None):
    """One block for one token at position ``pos``.

    W: dict with fp64 matrices wq [H*D][d], wk, wv [Hkv*D][d], wo [d][H*D], w_gate, w_up
       [F][d], w_down [d][F] -- the backbone's fp16 values or the river's q*s values.
    norms: dict with fp16 gains attn_norm [d], mlp_norm [d].
    K_l, V_l: this layer's cache for this row, [Hkv][Tmax][D]; slot ``pos`` is written.
    Returns h_out [d] fp16.
    """
    H, Hkv, D, eps, theta = cfg["H"], cfg["Hkv"], cfg["D"], cfg["eps"], cfg["theta"]
    a = rmsnorm(h_in16, norms["attn_norm"], eps)
    q = to_f16(_lin(W["wq"], a)).reshape(H, D)
    k = to_f16(_lin(W["wk"], a)).reshape(Hkv, D)
    v = to_f16(_lin(W["wv"], a)).reshape(Hkv, D)
    c, s = rope_cos_sin(pos, D, theta)
    q = apply_rope(q, c, s)
    k = apply_rope(k, c, s)
    K_l[:, pos, :] = k
    V_l[:, pos, :] = v
    o = decode_attention(q, K_l[:, : pos + 1, :], V_l[:, : pos + 1, :])
    h_mid = to_f16(h_in16.astype(F64) + to_f16(_lin(W["wo"], o.reshape(-1))).astype(F64))
    m = rmsnorm(h_mid, norms["mlp_norm"], eps)
    g = to_f16(_lin(W["w_gate"], m))
    u = to_f16(_lin(W["w_up"], m))
    a2 = to_f16(silu(g.astype(F64)) * u.astype(F64))
    h_out = to_f16(h_mid.astype(F64) + to_f16(_lin(W["w_down"], a2)).astype(F64))
    if trace is not None:
        trace.update(a=a, q=q, k=k, v=v, o=o, h_mid=h_mid, m=m, a2=a2)
    return h_out


def block_prefill(cfg, W, norms, H_in16, K_l, V_l):
    """One block over a whole prompt (positions 0..P-1) with causal attention.
    H_in16 [P][d]; writes K_l/V_l[:, 0:P]. Returns H_out [P][d] fp16."""
    H, Hkv, D, eps, theta = cfg["H"], cfg["Hkv"], cfg["D"], cfg["eps"], cfg["theta"]
    P = H_in16.shape[0]
    A = rmsnorm(H_in16, norms["attn_norm"], eps)
    Q = to_f16(_lin(W["wq"], A)).reshape(P, H, D)
    Kx = to_f16(_lin(W["wk"], A)).reshape(P, Hkv, D)
    Vx = to_f16(_lin(W["wv"], A)).reshape(P, Hkv, D)
    c, s = rope_cos_sin(np.arange(P), D, cfg["theta"])
    Q = apply_rope(Q, c[:, None, :], s[:, None, :])
    Kx = apply_rope(Kx, c[:, None, :], s[:, None, :])
    K_l[:, :P, :] = Kx.transpose(1, 0, 2)
    V_l[:, :P, :] = Vx.transpose(1, 0, 2)
    O = causal_attention(Q, K_l[:, :P, :], V_l[:, :P, :])
    Hm = to_f16(H_in16.astype(F64) + to_f16(_lin(W["wo"], O.reshape(P, H * D))).astype(F64))
    M = rmsnorm(Hm, norms["mlp_norm"], eps)
    G = to_f16(_lin(W["w_gate"], M))
    U = to_f16(_lin(W["w_up"], M))
    A2 = to_f16(silu(G.astype(F64)) * U.astype(F64))
    return to_f16(Hm.astype(F64) + to_f16(_lin(W["w_down"], A2)).astype(F64))


# --------------------------------------------------------------------------------------
# The model: backbone + river, prefill (sequence-level exit), decode (token-level exit)
# --------------------------------------------------------------------------------------

_MATS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


class RiverOracle:
    """Backbone (fp16 weights) plus its W4A16 river, driven token by token.

    weights: dict of fp16 numpy arrays: embed [V][d], lm_head [V][d] or None (tied to
    embed), final_norm [d], layers: list of L dicts with attn_norm, wq, wk, wv, wo,
    mlp_norm, w_gate, w_up, w_down.
    cfg keys: L, d, H, Hkv, D, F, V, eps, theta, group, entry (E_min), and optionally
    zero_point (True: the river uses the zero-point format of reading R5z).
    ``layers`` restricts which layers are materialised (for per-layer slices of a
    large model); the others must not be run. ``river_layers`` (default: ``layers``)
    restricts the river copies separately, so a run whose exit layers are known ahead
    holds only the backbone blocks it runs and the river blocks it runs.
    """

    def __init__(self, cfg, weights, layers=None, river_layers=None):
        self.cfg = dict(cfg)
        self.cfg.setdefault("entry", 1)
        self.L = cfg["L"]
        self.w16 = weights
        idx = range(self.L) if layers is None else layers
        ridx = idx if river_layers is None else river_layers
        self.bb = {}
        self.rv = {}
        self.qcodes = {}
        for i in idx:
            lw = weights["layers"][i]
            self.bb[i] = {m: np.asarray(lw[m]).astype(F64) for m in _MATS}
        zp = bool(self.cfg.get("zero_point", False))  # reading R5z instead of R5
        for i in ridx:
            lw = weights["layers"][i]
            self.rv[i] = {}
            self.qcodes[i] = {}
            for m in _MATS:
                if zp:
                    q, s, z = quantize_w4_zp(lw[m], cfg["group"])
                    self.qcodes[i][m] = (q, s, z)
                    self.rv[i][m] = dequantize_w4_zp(q, s, z, cfg["group"])
                else:
                    q, s = quantize_w4(lw[m], cfg["group"])
                    self.qcodes[i][m] = (q, s)
                    self.rv[i][m] = dequantize_w4(q, s, cfg["group"])
        self.embed16 = np.asarray(weights["embed"], dtype=F16)
        head = weights.get("lm_head")
        self.head16 = self.embed16 if head is None else np.asarray(head, dtype=F16)
        self._head64 = None

    # -- pieces -------------------------------------------------------------------------
    def norms(self, i):
        lw = self.w16["layers"][i]
        return {"attn_norm": lw["attn_norm"], "mlp_norm": lw["mlp_norm"]}

    def weights_for(self, i, river):
        return self.rv[i] if river else self.bb[i]

    def head_logits(self, h16):
        """Original fp16 LM head on the final-normed state ([paperlayer] §4 Inference with
        Seamless Exit). h16 [..., d] -> logits [..., V] fp64."""
        if self._head64 is None:
            self._head64 = self.head16.astype(F64)
        x = rmsnorm(h16, self.w16["final_norm"], self.cfg["eps"])
        return x.astype(F64) @ self._head64.T

    def new_kv(self, B, Tmax):
        c = self.cfg
        return OracleKV(c["L"], B, c["Hkv"], Tmax, c["D"])

    # -- exit rule (token level, [aitrends] exit criterion; [paperlayer] §4) ------------
    def _decide(self, l, s, forced, tau, gpu_exit, margin):
        """Exit after backbone layer l (1-based)?"""
        if forced is not None:
            return l == int(forced)
        if l < self.cfg["entry"]:
            return False
        if gpu_exit is not None and abs(s - tau) <= margin:
            return int(gpu_exit) == l
        return s > tau

    def decode_step(self, kv, tokens, forced_exit=None, tau=None, gpu_exit=None,
                    margin=1e-3, keep_hidden=True):
        """One generated token per row at position kv.pos[b].

        forced_exit [B] (exit after backbone layer e; e = L never exits; e = 0 runs no backbone
        block at all: every block on the river, the pages' "Full Quantization" comparator of
        [paperlayer] §5) or tau (with the GPU's exit_layer [B] used only where |s - tau| <=
        margin).
        Returns dict: tokens [B], logits [B][V] fp64, exit_layer [B], sim [B][L] (s(l) at
        index l-1, NaN where not computed), hs [L+1][B][d] fp16 (hs[0] = embedding row).
        """
        if forced_exit is None and tau is None:
            raise ValueError("decode_step needs forced_exit or tau")
        c = self.cfg
        L = self.L
        B = len(tokens)
        out_tok = np.zeros(B, dtype=np.int64)
        logits = np.zeros((B, c["V"]), dtype=F64)
        exit_layer = np.full(B, L, dtype=np.int64)
        sim = np.full((B, L), np.nan, dtype=F64)
        hs = np.zeros((L + 1, B, c["d"]), dtype=F16) if keep_hidden else None
        for b in range(B):
            pos = int(kv.pos[b])
            h = self.embed16[int(tokens[b])].copy()
            if keep_hidden:
                hs[0, b] = h
            exited = forced_exit is not None and int(forced_exit[b]) == 0
            if exited:
                exit_layer[b] = 0
            for l in range(1, L + 1):
                W = self.weights_for(l - 1, exited)
                h_new = block_decode(c, W, self.norms(l - 1), h, pos,
                                     kv.K[l - 1, b], kv.V[l - 1, b])
                kv.count[l - 1, b, pos] += 1
                if not exited and l < L:
                    s = np.nan
                    if forced_exit is None and l >= c["entry"]:
                        s = cosine(h, h_new)
                        sim[b, l - 1] = s
                    f = None if forced_exit is None else forced_exit[b]
                    g = None if gpu_exit is None else gpu_exit[b]
                    if self._decide(l, s, f, tau, g, margin):
                        exited = True
                        exit_layer[b] = l
                h = h_new
                if keep_hidden:
                    hs[l, b] = h
            lg = self.head_logits(h)
            logits[b] = lg
            out_tok[b] = argmax_lowest(lg)
            kv.pos[b] = pos + 1
        return {"tokens": out_tok, "logits": logits, "exit_layer": exit_layer,
                "sim": sim, "hs": hs}

    def prefill(self, kv, tokens, prefill_exit=None, tau=None, gpu_seq_exit=None,
                margin=1e-3, keep_hidden=False):
        """Prompt tokens [B][P] at positions 0..P-1 with a sequence-level exit
        ([paperlayer] §4 Inference with Seamless Exit; §3 Sequence-level Exit).

        Forced mode: every row exits after backbone layer ``prefill_exit``. Tau mode: row b
        exits after backbone layer l (entry <= l < L) iff min over its tokens of
        s_t(l) > tau (reading R8); inside the margin the GPU's seq_exit decides.
        Returns dict: tokens [B] (first generated token), logits [B][V] at position P-1,
        seq_exit [B], min_sim [B][L], hs (optional) [L+1][B][P][d].
        """
        if prefill_exit is None and tau is None:
            raise ValueError("prefill needs prefill_exit or tau")
        c = self.cfg
        L = self.L
        tokens = np.asarray(tokens)
        B, P = tokens.shape
        out_tok = np.zeros(B, dtype=np.int64)
        logits = np.zeros((B, c["V"]), dtype=F64)
        seq_exit = np.full(B, L, dtype=np.int64)
        min_sim = np.full((B, L), np.nan, dtype=F64)
        hs = np.zeros((L + 1, B, P, c["d"]), dtype=F16) if keep_hidden else None
        for b in range(B):
            Hs = self.embed16[tokens[b]].copy()
            if keep_hidden:
                hs[0, b] = Hs
            exited = False
            for l in range(1, L + 1):
                W = self.weights_for(l - 1, exited)
                Hn = block_prefill(c, W, self.norms(l - 1), Hs, kv.K[l - 1, b], kv.V[l - 1, b])
                kv.count[l - 1, b, :P] += 1
                if not exited and l < L:
                    s = np.nan
                    if prefill_exit is None and l >= c["entry"]:
                        s = min(cosine(Hs[t], Hn[t]) for t in range(P))
                        min_sim[b, l - 1] = s
                    g = None if gpu_seq_exit is None else gpu_seq_exit[b]
                    if self._decide(l, s, prefill_exit, tau, g, margin):
                        exited = True
                        seq_exit[b] = l
                Hs = Hn
                if keep_hidden:
                    hs[l, b] = Hs
            lg = self.head_logits(Hs[P - 1])
            logits[b] = lg
            out_tok[b] = argmax_lowest(lg)
            kv.pos[b] = P
        return {"tokens": out_tok, "logits": logits, "seq_exit": seq_exit,
                "min_sim": min_sim, "hs": hs}
