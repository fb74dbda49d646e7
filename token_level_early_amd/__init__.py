"""River-LLM token-level early-exit decode for MI355X (gfx950).

The compute path is the C-ABI library ``libriver.so`` (HIP kernels, built from
``csrc/``); ``river`` is its thin ctypes binding. Importing this package loads
nothing; ``river.load()`` opens the library and fails loudly if it is missing.
"""

__all__ = ["configs", "synth", "river"]
