"""CPU oracle for River-LLM token-level early-exit decode.

TEST INFRASTRUCTURE ONLY. Nothing in the product package (``token_level_early_amd``)
imports, links or runs anything under ``oracle/``. The only callers are ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``.

The oracle is plain NumPy, written from the method's description; it shares no code,
tables or helpers with the HIP path. See ``river_oracle`` for the per-function
citations and the list of readings taken where the pages leave a step open.
"""

from .river_oracle import (  # noqa: F401
    to_f16,
    quantize_w4,
    quantize_w4_zp,
    dequantize_w4_zp,
    pack_codes,
    pack_nibbles,
    unpack_nibbles,
    dequantize_w4,
    rmsnorm,
    rope_cos_sin,
    apply_rope,
    cosine,
    silu,
    decode_attention,
    causal_attention,
    block_decode,
    block_prefill,
    OracleKV,
    RiverOracle,
    argmax_lowest,
)
