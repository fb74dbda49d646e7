"""Algorithmic HBM bytes of one early-exit decode step (what the method must move per token).

Each layer's weights are read once on the path the token takes -- never the alternative --
plus the shared KV cache read and the one-slot append, the embedding row, the final norm and
the fp16 LM head:

    B_tok = sum_l [e >= l ? W16 : W4] + L*kv*(pos+1) + L*kv + 2d + 2d + 2*V*d
    W16 = 2*P_l + 4d          (fp16 matrices + two RMSNorm gain vectors)
    W4  = P_l/2 + 2*P_l/g + 4d (int4 nibbles + one fp16 scale per group + gains), plus P_l/g
                              (one zero-point byte per group) in the zero-point format
    kv  = 2*Hkv*D*2           (K and V of one position, fp16)

Activation vectors (a few KB per kernel) are not counted.
"""


def op_params(c):
    """Parameters of the decode-step GEMVs: {op: (N, K)}."""
    d, H, Hkv, D, F = c["d"], c["H"], c["Hkv"], c["D"], c["F"]
    return {"qkv": ((H + 2 * Hkv) * D, d), "o": (d, H * D), "gu": (2 * F, d), "down": (d, F)}


def matrix_bytes(N, K, river, group, zero_point=False):
    if river:
        ng = N * ((K + group - 1) // group)
        return N * K // 2 + ng * 2 + (ng if zero_point else 0)
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
    b = matrix_bytes(N, K, river, g, c.get("zero_point", False))
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


def batch_step_bytes(c, exits, positions):
    """Algorithmic bytes of one batched decode step: row b exits after e_b backbone layers and
    runs at position p_b. At layer l the backbone matrices (and norm gains) are read once if any
    row runs l on the backbone, the river copy once if any row has exited; every row reads its
    own K/V of positions 0..p_b and appends one slot; each row reads its embedding row; the
    final norm and the LM head are read once for all rows."""
    L, d = c["L"], c["d"]
    kv = 2 * c["Hkv"] * c["D"] * 2
    total = 0
    for l in range(1, L + 1):
        for river, used in ((False, any(e >= l for e in exits)), (True, any(e < l for e in exits))):
            if used:
                total += sum(matrix_bytes(N, K, river, c["group"], c.get("zero_point", False))
                             for N, K in op_params(c).values())
                total += 4 * d  # attention and MLP norm gains
    for p in positions:
        total += L * kv * (p + 1) + L * kv + 2 * d
    total += 2 * d + 2 * c["V"] * d
    return total


def batch_op_bytes(c, op, exits, layer, positions):
    """Algorithmic bytes of one batched launch of `op` at `layer` (see batch_step_bytes): the
    matrices of each weight stream some row uses at that layer (with that stream's norm gains
    for qkv and gu), plus each row's K/V append (qkv) or K/V read (attn); lm: head + final norm."""
    d = c["d"]
    kv = 2 * c["Hkv"] * c["D"] * 2
    if op == "attn":
        return sum(kv * (p + 1) for p in positions)
    if op == "lm":
        return 2 * c["V"] * d + 2 * d
    N, K = op_params(c)[op]
    total = 0
    for river, used in ((False, any(e >= layer for e in exits)), (True, any(e < layer for e in exits))):
        if used:
            total += (matrix_bytes(N, K, river, c["group"], c.get("zero_point", False))
                      + (2 * d if op in ("qkv", "gu") else 0))
    if op == "qkv":
        total += kv * len(exits)
    return total
