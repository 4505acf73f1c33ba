"""io_aware_kv_amd: the IO-aware fused KV-cache step of a diffusion LLM
attention layer (Flash-dLLM), as hand-written HIP kernels for MI355X (gfx950)
behind a C ABI.  The Python side is a thin ctypes binding (``binding``) plus
seeded input generators (``workloads``)."""
