"""Model shapes and decode workloads (synthetic, seeded).

Each entry names a Llama-style decoder shape and one decode workload on it. The
method-level fields (``group``, ``entry``) follow the river construction: int4
weights, one fp16 scale per ``group`` input columns, exit tests from layer
``entry`` onward.
"""

TINY = dict(
    name="tiny", cfg_id=0,
    L=4, d=256, H=4, Hkv=2, D=64, F=688, V=1024, tied=False,
    eps=1e-5, theta=10000.0, group=64, entry=1,
    batch=1, prompt=64, steps=32,
    tau=0.95, forced_exit=2,
)

LLAMA_1B = dict(
    name="llama3.2-1b-shape", cfg_id=1,
    L=16, d=2048, H=32, Hkv=8, D=64, F=8192, V=128256, tied=True,
    eps=1e-5, theta=500000.0, group=128, entry=1,
    batch=1, prompt=512, steps=256,
    # tau is calibrated by bisection on the seeded inputs so that about half of the
    # decode tokens exit by layer 8.
    tau=None, exit_by=8, exit_frac=0.5,
)

LLAMA_8B = dict(
    name="llama3.1-8b-shape", cfg_id=2,
    L=32, d=4096, H=32, Hkv=8, D=128, F=14336, V=128256, tied=False,
    eps=1e-5, theta=500000.0, group=128, entry=1,
    batch=1, prompt=2048, steps=256,
    # forced exit layer per decode token, uniform on {8..20} (mean 14)
    sched=("uniform", 8, 20),
)

LLAMA_8B_BS16 = dict(LLAMA_8B, name="llama3.1-8b-shape-bs16", cfg_id=3,
                     batch=16, prompt=4096, steps=128, sched=("uniform", 8, 32))

LLAMA_8B_64K = dict(LLAMA_8B, name="llama3.1-8b-shape-64k", cfg_id=4,
                    batch=1, prompt=65536, steps=64, sched=("half", 8, 20))

# The same workloads with the zero-point river format (scale and zero point per group).
TINY_ZP = dict(TINY, name="tiny-zp", zero_point=True)
LLAMA_8B_ZP = dict(LLAMA_8B, name="llama3.1-8b-shape-zp", zero_point=True)

ALL = {c["name"]: c for c in (TINY, LLAMA_1B, LLAMA_8B, LLAMA_8B_BS16, LLAMA_8B_64K, TINY_ZP, LLAMA_8B_ZP)}


def model_cfg(c):
    """The subset of fields that defines the model (what the oracle and the library need)."""
    keys = ("L", "d", "H", "Hkv", "D", "F", "V", "tied", "eps", "theta", "group", "entry")
    out = {k: c[k] for k in keys}
    out["zero_point"] = bool(c.get("zero_point", False))
    return out
