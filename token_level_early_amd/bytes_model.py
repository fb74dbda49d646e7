"""Algorithmic HBM bytes of one early-exit decode step (what the method must move per token).

Each layer's weights are read once on the path the token takes -- never the alternative --
plus the shared KV cache read and the one-slot append, the embedding row, the final norm and
the fp16 LM head:

    B_tok = sum_l [e >= l ? W16 : W4] + L*kv*(pos+1) + L*kv + 2d + 2d + 2*V*d
    W16 = 2*P_l + 4d          (fp16 matrices + two RMSNorm gain vectors)
    W4  = P_l/2 + 2*P_l/g + 4d (int4 nibbles + one fp16 scale per group + gains)
    kv  = 2*Hkv*D*2           (K and V of one position, fp16)

Activation vectors (a few KB per kernel) are not counted.
"""


def op_params(c):
    """Parameters of the decode-step GEMVs: {op: (N, K)}."""
    d, H, Hkv, D, F = c["d"], c["H"], c["Hkv"], c["D"], c["F"]
    return {"qkv": ((H + 2 * Hkv) * D, d), "o": (d, H * D), "gu": (2 * F, d), "down": (d, F)}


def matrix_bytes(N, K, river, group):
    if river:
        return N * K // 2 + N * ((K + group - 1) // group) * 2
    return 2 * N * K


def op_bytes(c, op, river=False, pos=0):
    """Algorithmic bytes of one launch of `op` for one row: op in qkv, attn, o, gu, down, lm.
    qkv includes the attention RMSNorm gains and the KV append; gu the MLP norm gains; attn
    reads K and V of positions 0..pos; lm the final norm gains and the LM head."""
    d, g = c["d"], c["group"]
    kv = 2 * c["Hkv"] * c["D"] * 2
    if op == "attn":
        return kv * (pos + 1)
    if op == "lm":
        return 2 * c["V"] * d + 2 * d
    N, K = op_params(c)[op]
    b = matrix_bytes(N, K, river, g)
    if op == "qkv":
        b += 2 * d + kv
    if op == "gu":
        b += 2 * d
    return b


def layer_bytes(c, river):
    return sum(op_bytes(c, o, river) for o in ("qkv", "o", "gu", "down")) - 2 * c["Hkv"] * c["D"] * 2


def token_bytes(c, e, pos):
    """Bytes of one decode token with exit layer e at position pos (0-based)."""
    L = c["L"]
    total = 2 * c["d"]  # embedding row
    for l in range(1, L + 1):
        river = l > e
        for o in ("qkv", "o", "gu", "down"):
            total += op_bytes(c, o, river)
        total += op_bytes(c, "attn", pos=pos)
    total += op_bytes(c, "lm")
    return total
