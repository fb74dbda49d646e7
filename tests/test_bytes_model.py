"""The algorithmic byte model used for the roofline figures (no GPU): closed-form cases."""

from token_level_early_amd import bytes_model as bm
from token_level_early_amd import configs

def test_batch_byte_model_reduces_to_the_single_row_model():
    c = configs.model_cfg(configs.LLAMA_8B)
    for e, p in ((14, 2176), (32, 100), (1, 0)):
        assert bm.batch_step_bytes(c, [e], [p]) == bm.token_bytes(c, e, p)
        # one row: the per-launch model sums to the step model
        ops = sum(bm.batch_op_bytes(c, o, [e], l, [p]) for l in range(1, c["L"] + 1)
                  for o in ("qkv", "attn", "o", "gu", "down"))
        assert ops + bm.batch_op_bytes(c, "lm", [e], 0, [p]) + 2 * c["d"] == bm.token_bytes(c, e, p)
    # identical rows read the weights once: only KV, appends and embedding rows scale with B
    one = bm.batch_step_bytes(c, [14], [1000])
    four = bm.batch_step_bytes(c, [14] * 4, [1000] * 4)
    kv = 2 * c["Hkv"] * c["D"] * 2
    assert four - one == 3 * (c["L"] * kv * 1001 + c["L"] * kv + 2 * c["d"])
    # rows that disagree at a layer read both copies there
    both = bm.batch_step_bytes(c, [8, 32], [0, 0]) - bm.batch_step_bytes(c, [32, 32], [0, 0])
    w4 = sum(bm.matrix_bytes(N, K, True, c["group"]) for N, K in bm.op_params(c).values()) + 4 * c["d"]
    assert both == 24 * w4


def test_byte_model_matches_hand_derived_per_layer_figures():
    """8B per-layer weight bytes worked out by hand from the Llama-3.1-8B shape
    (P_l = 218,103,808 parameters per block): 2*P_l + 4d = 436.22 MB fp16, P_l/2 + 2*P_l/128
    + 4d = 112.48 MB int4 + scales (group 128); LM head 2*V*d = 1.051 GB."""
    c = configs.model_cfg(configs.LLAMA_8B)
    d = c["d"]
    w16 = sum(bm.matrix_bytes(N, K, False, 128) for N, K in bm.op_params(c).values()) + 4 * d
    w4 = sum(bm.matrix_bytes(N, K, True, 128) for N, K in bm.op_params(c).values()) + 4 * d
    assert round(w16 / 1e6, 2) == 436.22
    assert round(w4 / 1e6, 2) == 112.48
    assert round(bm.op_bytes(c, "lm") / 1e9, 3) == 1.051


def test_zero_point_format_adds_one_byte_per_group():
    """The zero-point river reads one more byte per group: P_l/128 = 1.70 MB per 8B block."""
    c = configs.model_cfg(configs.LLAMA_8B)
    cz = configs.model_cfg(configs.LLAMA_8B_ZP)
    P_l = 218_103_808
    assert bm.token_bytes(cz, 0, 100) - bm.token_bytes(c, 0, 100) == c["L"] * P_l // 128
    assert bm.token_bytes(cz, c["L"], 100) == bm.token_bytes(c, c["L"], 100)
