"""KDA state recurrence on MI355X (gfx950): chunked prefill with checkpoints,
decode, verify-and-replay and head packing, as hand-written HIP kernels behind
a C ABI (include/kda.h).  This package holds the thin Python binding
(``linear_attention_recurrence_kda_amd.kda``), the build step and the seeded
input generators.  Importing the package does not load the library; the
binding does, and fails loudly when the library is missing.
"""

__all__ = ["kda", "inputs", "build"]
