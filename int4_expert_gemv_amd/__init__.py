"""int4/int8 quantized expert GEMV and MoE expert FFN for MI355X (gfx950).

The compute lives in libqmoe.so (hand-written HIP kernels behind a C ABI,
declared in include/qmoe.h).  `int4_expert_gemv_amd.qmoe` is the thin ctypes
binding with the same entry-point names; `int4_expert_gemv_amd.synth` holds
the seeded synthetic-input generators.
"""
